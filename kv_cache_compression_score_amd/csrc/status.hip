// Status strings of the kvcc C ABI.
#include "common.hpp"

extern "C" const char* kv_status_string(int status) {
  switch (status) {
    case KV_OK: return "ok";
    case KV_ERR_NULL: return "a required pointer is NULL";
    case KV_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case KV_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KV_ERR_DTYPE: return "unsupported dtype";
    case KV_ERR_MODE: return "unknown budget mode or out-of-range budget value";
    case KV_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}
