"""MI355X-native KV-cache scoring, selection, compaction and decode attention.

The four steps run in the HIP library ``libkvcc.so`` (built from ``csrc/``);
``api`` marshals torch device tensors into its C entry points.  Importing the
package loads nothing; the library is loaded on first use and its absence is
an error, never a fallback.
"""
