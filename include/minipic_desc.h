/*
 * Host-side descriptor builder and block cache for position-free paged
 * attention (no GPU code; plain host memory).
 *
 * From one request's token ids with the user-facing markers of "MiniPIC:
 * Flexible Position-Independent Caching in <100LOC" (§3.1.1: SSep, PDep and
 * padding to a block boundary; §3.3.1 and §3.3.2 for how Block-Attention and
 * EPIC use them) this computes what minipic_prefill_attn needs per 16-token
 * block: a span id, the PDEP / GLOBAL flags, and the block's cache hash
 * following the hashing rule of §3.1.1:
 *   h_i = H(h_0, x_i)       if block i starts with SSep,
 *   h_i = H(h_0, x_<=i)     if block i starts with PDep,
 *   h_i = H(h_{i-1}, x_i)   otherwise,
 * where x_i are block i's tokens and h_0 the seed. A block cache maps hashes
 * to physical blocks so that a span (or a shared prefix) computed once is
 * reused by later requests at any offset.
 *
 * H is not fixed by the pages: here H(h, x) folds the tokens of x into h one
 * at a time with the SplitMix64 mixing function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", 2014):
 *   h <- mix(h ^ token + 0x9E3779B97F4A7C15).
 * A GLOBAL marker (an extension for a Prompt-Cache prefix, not one of the
 * pages' three primitives) sets the GLOBAL flag on its segment's blocks. Every
 * later token attends to GLOBAL blocks, so the K/V of a span that follows a
 * GLOBAL segment depend on it: a block that starts with SSep or GLOBAL hashes
 * as H(g, x_i), where g is the hash of the last GLOBAL block before it (h_0
 * when there is none). Without a GLOBAL segment this is the rule above.
 */
#ifndef MINIPIC_DESC_H
#define MINIPIC_DESC_H

#include <stdint.h>

#include "minipic.h"

#ifdef __cplusplus
extern "C" {
#endif

/* A marker token at a position that is not a block start (the padding
 * contract of §3.1.1 / §3.1.2 is broken); minipic_last_error() names it. */
#define MINIPIC_ERR_CONTRACT (-5)
/* The block cache has no free block left. */
#define MINIPIC_ERR_CACHE_FULL (-6)

/* Marker token ids; -1 disables a marker. */
typedef struct {
  int32_t ssep;
  int32_t pdep;
  int32_t global_;
  uint64_t seed;     /* h_0 */
} minipic_markers;

/*
 * Descriptors of one request's token sequence (host arrays).
 *   tokens[n]        : token ids in context order, markers included.
 *   block_size       : must be 16.
 *   hashes[max_blocks], span_id[max_blocks], flags[max_blocks] : outputs for
 *                      the ceil(n / 16) blocks (flags: MINIPIC_BLK_PDEP,
 *                      MINIPIC_BLK_GLOBAL). A segment runs from a marker block
 *                      to the next marker block; blocks before the first
 *                      marker form span 0 (e.g. a system prompt); span ids
 *                      count segments in order.
 *   num_blocks       : ceil(n / 16).
 * Returns MINIPIC_ERR_CONTRACT if a marker token is not the first token of a
 * block, MINIPIC_ERR_INVALID_ARG for NULL pointers, n < 0, block_size != 16
 * or max_blocks < ceil(n / 16). Outputs are not written on error.
 */
int minipic_describe_blocks(const int32_t* tokens, int64_t n, const minipic_markers* markers,
                            int32_t block_size, uint64_t* hashes, int32_t* span_id, uint8_t* flags,
                            int64_t max_blocks, int64_t* num_blocks);

/* Opaque hash -> physical block map over num_blocks physical blocks. */
typedef struct minipic_block_cache minipic_block_cache;

/* Returns NULL if num_blocks <= 0 or on allocation failure. */
minipic_block_cache* minipic_block_cache_create(int64_t num_blocks);
void minipic_block_cache_destroy(minipic_block_cache* cache);

/*
 * Physical blocks for one request's blocks (host arrays): a block whose hash
 * is cached reuses that physical block (hit[i] = 1: its K/V is already in the
 * cache); any other block takes a free physical block and is recorded under
 * its hash (hit[i] = 0: its tokens must be computed and written). Two equal
 * hashes in one request share one block. Writes block_table[nb], hit[nb] and
 * *num_hits. On MINIPIC_ERR_CACHE_FULL nothing is recorded.
 */
int minipic_block_cache_assign(minipic_block_cache* cache, const uint64_t* hashes, int64_t nb,
                               int32_t* block_table, uint8_t* hit, int64_t* num_hits);

/*
 * Slot mapping of the tokens of the blocks that missed: for every token t < n
 * whose block i has hit[i] == 0, slot = block_table[i] * 16 + t % 16, written
 * in token order to slots[]; the context indices of those tokens to
 * ctx_index[] (may be NULL). *count = the number of tokens written (<= n).
 */
int minipic_slot_mapping(const int32_t* block_table, const uint8_t* hit, int64_t n, int32_t block_size,
                         int64_t* slots, int32_t* ctx_index, int64_t* count);

#ifdef __cplusplus
}
#endif
#endif /* MINIPIC_DESC_H */
