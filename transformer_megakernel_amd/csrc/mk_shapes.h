// Model widths the decode kernel is compiled for.  The kernel is a template over these
// widths (every index is compile-time arithmetic), so a configuration must match one
// row: hidden, query heads, KV heads, head_dim, SwiGLU intermediate, and the number of
// K-chunks the down projection is consumed in.  Depth, vocabulary and cache length are
// free.  The article's model is Llama-3.2-1B; the down projection is split into 4
// chunks as in its MLP schedule wherever a quarter of the intermediate is a whole
// number of 1 KiB rows.
#pragma once

//        hidden  q  kv  hd   ffn   chunks
#define MK_SHAPES(X)                                                    \
  X(256, 4, 2, 64, 1024, 4)      /* tiny test decoder (512-byte rows) */ \
  X(512, 8, 2, 64, 2048, 4)      /* small test decoder (1 KiB rows)   */ \
  X(1024, 8, 2, 128, 3584, 1)    /* small test decoder, head_dim 128  */ \
  X(2048, 32, 8, 64, 8192, 4)    /* Llama-3.2-1B                      */ \
  X(4096, 32, 8, 128, 14336, 4)  /* Llama-3.1-8B                      */
