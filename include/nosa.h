/*
 * nosa.h -- C ABI of libnosa, the decode-time hot path of NOSA (Native and
 * Offloadable Sparse Attention, arXiv 2510.13602) on AMD CDNA4 (gfx950).
 *
 * The path, per decode step and per (batch b, KV head h):
 *   1. nosa_pool_keys          compressed keys and block eviction scores
 *   2. nosa_select_blocks      query-aware top-kq U query-agnostic top-ke
 *   3. nosa_fetch_blocks       HBM block pool: set difference, slot choice,
 *                              host -> HBM gather of the missing blocks
 *   4. nosa_sparse_decode_attn exact attention over the selected blocks plus
 *                              the current (window) block
 * and the same steps in fewer launches: nosa_decode_step (2 + 4 for a cache
 * resident in HBM, one launch; nosa_decode_step_static without a
 * workspace), nosa_select_update_pool (2 + the table part of 3) and
 * nosa_sparse_decode_attn_fetch (the gather of 3 + 4) for an offloaded cache,
 * or 3 split around a side stream (nosa_update_pool, nosa_gather_blocks,
 * nosa_sparse_decode_attn_pool); per-entry pooling (nosa_pool_keys_entries);
 * prefill chunks (nosa_sparse_chunk_attn, nosa_select_blocks_shared); the
 * step before 1 (nosa_split_qkv); and two alternative readings kept for
 * comparison (nosa_select_blocks_fill, nosa_sparse_decode_attn_bias).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tokens are grouped in blocks of NOSA_BLOCK = 64 and sub-blocks of
 *   NOSA_SUB = 16 (the NOSA-1B release post, "工程实现亮点": block size and
 *   top-K are both 64; the 16-token sub-block is this library's choice).
 * - Element type: NOSA_BF16 (bfloat16) or NOSA_F32; head_dim 64 or 128;
 *   n_q_heads a multiple of n_kv_heads with at most 16 query heads per KV
 *   head.
 * - KV block format (one block = 2*64*head_dim elements): the 64 keys,
 *   then the 64 values, each half stored as 1 KiB MFMA fragments of 64 lanes
 *   x 16 bytes, so that the attention reads every fragment with one
 *   contiguous wavefront load.  With tile_token(t, r) = 32(t/2) + 8(r/4) +
 *   4(t%2) + r%4 and lane = 16g + r (g < 4, r < 16):
 *     bf16: key fragment t*(D/32)+s holds, in lane 16g+r, K[tile_token(t,r)]
 *           [32s+8g .. 32s+8g+7]  (t < 4, s < D/32); value fragment
 *           h*(D/16)+u holds V[32h+8g .. 32h+8g+7][16u+r]  (h < 2, u < D/16);
 *     fp32: key fragment t*(D/16)+s holds K[16t+r][16s+4g .. 16s+4g+3];
 *           value fragment t*(D/16)+u holds V[16t+4g .. 16t+4g+3][16u+r].
 *   The cache of one layer is [B][Hkv][max_blocks][block]; the HBM pool is
 *   [B][Hkv][pool_slots][block].  Host and HBM use the same format, so a
 *   block moves as one contiguous span (32 KiB at D=128 bf16).
 * - Decode position p attends tokens [0, p]; its window is block c = p/64
 *   (tokens 64c..p); the candidates for selection are blocks 0..c-1.
 * - Every buffer is allocated and owned by the caller.  "device" means HBM
 *   of the current device; "pinned host" means host memory the GPU can read
 *   directly (hipHostMalloc).  The library allocates nothing, frees nothing
 *   and never synchronises: each call enqueues its kernels on `stream`
 *   (a hipStream_t; NULL = the default stream) and returns.
 * - Errors: every argument is validated on the host before any launch; a
 *   failed call launches nothing.  Return codes below; nosa_last_error()
 *   gives the text of the last failure on the calling thread.  Values that
 *   live in device memory (positions, selected ids, slots) cannot be checked
 *   on the host: the kernels skip out-of-range entries instead of reading or
 *   writing outside the buffers, as documented per call.
 * - Reentrant: concurrent calls are safe when their streams, outputs and
 *   workspaces are distinct.
 */
#ifndef NOSA_H
#define NOSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NOSA_BLOCK 64
#define NOSA_SUB 16

enum nosa_dtype { NOSA_BF16 = 0, NOSA_F32 = 1 };

enum nosa_status {
  NOSA_OK = 0,
  NOSA_ERR_ARG = -1,          /* null pointer, bad size or range */
  NOSA_ERR_UNSUPPORTED = -2,  /* dtype, head_dim or group size not built */
  NOSA_ERR_HIP = -3,          /* a HIP launch or runtime call failed */
  NOSA_ERR_WORKSPACE = -4     /* workspace smaller than nosa_workspace_size() */
};

enum nosa_op { NOSA_OP_SELECT = 1, NOSA_OP_ATTN = 2, NOSA_OP_STEP = 3 };

typedef struct nosa_dims {
  int32_t batch;       /* B */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; G = Hq / Hkv query heads share one KV head */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t max_blocks;  /* NB: capacity of the cache in 64-token blocks per (b, h) */
  int32_t dtype;       /* enum nosa_dtype */
} nosa_dims;

/*
 * nosa_split_qkv -- split one fused QKV projection output per token into the
 * path's inputs, with the eviction head fused in.
 *
 * NOSI fuses the eviction heads with the QKV split into one kernel (montaan
 * summary, "System Optimization (NOSI)" item 1); the head is Eq. 4 of the
 * same summary ("Key Design Components" item 3): s^e = softplus(v W1) W2,
 * one score per KV pair from its value, used as the eviction logit that
 * nosa_pool_keys averages.  For token t of batch entry b at p = pos[b][t]:
 *   q_out[b][t] = the query heads;  the key and value rows of every KV head
 *   h go to block p/64, token p%64, of the cache (fragment format);
 *   evict_logits[b][h][p] = sum_j softplus(sum_d v[d] W1[h][d][j]) W2[h][j]
 *   (fp32 products and sums; the order of the sums is the kernel's).
 *
 *   qkv           device [B][n_tok][(Hq + 2 Hkv) * D], cache dtype: the
 *                 query heads, then the key heads, then the value heads
 *   pos           device int32 [B][n_tok]; tokens outside [0, NB*64) only
 *                 have their query copied
 *   w1, w2        device fp32 [Hkv][D][d_e], [Hkv][d_e]  (1 <= d_e <= 512)
 *   q_out         device [B][n_tok][Hq][D], cache dtype            (written)
 *   kv            device cache [B][Hkv][NB][block]           (written rows)
 *   evict_logits  device fp32 [B][Hkv][NB*64]                (written rows)
 * Errors: -1 for NULL buffers or n_tok outside [1, 65535]; -2 for d_e
 * outside [1, 512], batch above 65535 or more than 16 KV heads.
 */
int nosa_split_qkv(const nosa_dims* dims, const void* qkv, int32_t n_tok, const int32_t* pos,
                   const float* w1, const float* w2, int32_t d_e, void* q_out, void* kv,
                   float* evict_logits, void* stream);

/*
 * nosa_pool_keys -- compressed keys and the block eviction score.
 *
 * Defined by the gist.science summary of NOSA ("1. Algorithme : NOSA",
 * block implementation: mean pooling inside sub-blocks, then max pooling per
 * block, for the selection scores) and the montaan summary ("Key Design
 * Components" item 2).  For every (b, h) and every block j in
 * [blk_begin, blk_end), sub-blocks s = 4j..4j+3:
 *   k_comp[b][h][s][:] = (sum of the 16 keys of s, fp32, token order) / 16,
 *                        rounded to nearest-even to the cache dtype;
 *   e_sub[b][h][s]     = (sum of the 16 logits of s, fp32, token order) / 16;
 *   e_blk[b][h][j]     = max(e_sub[b][h][4j .. 4j+3]).
 * Results are bit-exact (fixed summation order).
 *
 *   kv            device  blocks in the library's block format; block j of
 *                         (b, h) starts at element
 *                         (b*Hkv + h) * kv_unit_stride + j * kv_block_stride
 *                         (the cache [B][Hkv][NB][block]: strides NB*block and
 *                         block; a window buffer [B][Hkv][block] holding one
 *                         block: strides block and 0).  Only keys are read.
 *   evict_logits  device  fp32 [B][Hkv][NB*64]  per-token eviction logits
 *                         (pre-exponential, as ED-DMA selects on them)
 *   blk_begin, blk_end    0 <= blk_begin <= blk_end <= NB (host ints)
 *   k_comp        device  [B][Hkv][NB*4][D], cache dtype      (written)
 *   e_sub         device  fp32 [B][Hkv][NB*4]                 (written)
 *   e_blk         device  fp32 [B][Hkv][NB]                   (written)
 * Only the entries of blocks in the range are written.
 */
int nosa_pool_keys(const nosa_dims* dims, const void* kv, int64_t kv_unit_stride,
                   int64_t kv_block_stride, const float* evict_logits, int32_t blk_begin,
                   int32_t blk_end, void* k_comp, float* e_sub, float* e_blk, void* stream);

/*
 * nosa_pool_keys_entries -- nosa_pool_keys for one block per batch entry,
 * the block named on the device.
 *
 * The sequences of a batch sit at their own positions, so their windows
 * complete blocks on different steps; NOSI's memory manager handles each
 * sequence's blocks as units of its own (montaan summary, "System
 * Optimization (NOSI)" item 2).  For every b with 0 <= entry_block[b] < NB
 * and every KV head h, block j = entry_block[b] of (b, h) is pooled exactly
 * as nosa_pool_keys pools it (same formulas, same bit-exact results); entries
 * with any other value are skipped and nothing of theirs is written.
 *
 *   entry_block   device int32 [B]    (read; the caller's, not kept)
 *   kv, strides   as for nosa_pool_keys: block j of (b, h) starts at element
 *                 (b*Hkv + h) * kv_unit_stride + j * kv_block_stride; a
 *                 window buffer [B][Hkv][block] holding each entry's just
 *                 completed block has strides block and 0
 *   evict_logits, k_comp, e_sub, e_blk    as for nosa_pool_keys
 * Errors: -1 for a NULL entry_block or buffer, or negative strides.  The
 * block indices are read on the device, so one launch serves any mix of
 * entries (a graph can hold it).
 */
int nosa_pool_keys_entries(const nosa_dims* dims, const void* kv, int64_t kv_unit_stride,
                           int64_t kv_block_stride, const float* evict_logits,
                           const int32_t* entry_block, void* k_comp, float* e_sub, float* e_blk,
                           void* stream);

/*
 * nosa_select_blocks -- the blocks each query row attends (Eq. 7).
 *
 * Defined by the montaan summary ("How it works": one Top-k over the query
 * scores and one over the eviction-head scores; "Key Design Components"
 * item 4, Eq. 7: up to k blocks, query-aware budget kq first, the
 * query-agnostic budget ke for the rest) and the gist.science summary (dual
 * selection Gamma_q / Gamma_e; ED-DMA: select on pre-exponential scores).
 * For query row r of batch b at position p = pos[b][r], with c = p / 64:
 *   qsum      = sum of the G query heads of KV head h (fp32);
 *   sigma_s   = qsum . k_comp[b][h][s]   for sub-blocks s < 4c (fp32);
 *   score_j   = max(sigma_4j .. sigma_4j+3)              (no scale, no exp);
 *   Gamma_q   = the min(kq, c) blocks j < c with the best (score desc, j asc);
 *   Gamma_e   = the min(ke, c) blocks j < c with the best (e_blk desc, j asc);
 *   sel[b][r][h][0 .. n-1] = Gamma_q U Gamma_e ascending, the rest -1;
 *   n_sel[b][r][h] = n (<= kq + ke).
 * The window block c is not part of sel: the attention always adds it.
 *
 *   q        device  [B][n_query][Hq][D], cache dtype
 *   n_query  query rows per batch entry (1 for decode)
 *   pos      device  int32 [B][n_query]; rows with pos < 0 or
 *                    pos >= NB*64 get n_sel = 0
 *   k_comp, e_blk    as written by nosa_pool_keys for blocks 0..c-1
 *   kq, ke   >= 0 budgets (in blocks)
 *   sel      device  int32 [B][n_query][Hkv][kq+ke]            (written)
 *   n_sel    device  int32 [B][n_query][Hkv]                    (written)
 *   ws       device  workspace of at least
 *                    nosa_workspace_size(dims, NOSA_OP_SELECT, n_query, kq, ke)
 *                    bytes, zero-filled once before its first use; every
 *                    call leaves it ready for the next one.
 */
int nosa_select_blocks(const nosa_dims* dims, const void* q, int32_t n_query,
                       const int32_t* pos, const void* k_comp, const float* e_blk,
                       int32_t kq, int32_t ke, int32_t* sel, int32_t* n_sel, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * nosa_select_blocks_fill -- nosa_select_blocks under the other reading of
 * Eq. 7, a variant kept for comparison (the path itself uses the union of
 * two independent top-k sets).
 *
 * The montaan summary's Eq. 7 ("Key Design Components" item 4) fills "the
 * remainder" with query-agnostic blocks; read as the remainder of the
 * candidates, the query-agnostic part is the top-ke of e_blk over the
 * candidates outside Gamma_q:
 *   Gamma_q  as in nosa_select_blocks;
 *   F        = the min(ke, c - |Gamma_q|) blocks j < c, j not in Gamma_q, with
 *              the best (e_blk desc, j asc);
 *   sel      = Gamma_q U F ascending, exactly min(kq + ke, c) blocks.
 * A block can leave F when it enters Gamma_q and come back when it leaves
 * Gamma_q, which the eviction rule of the same summary (item 1) forbids.
 * Arguments, layouts, workspace and errors as nosa_select_blocks.
 */
int nosa_select_blocks_fill(const nosa_dims* dims, const void* q, int32_t n_query,
                            const int32_t* pos, const void* k_comp, const float* e_blk,
                            int32_t kq, int32_t ke, int32_t* sel, int32_t* n_sel, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * nosa_select_blocks_shared -- one selection for all n_query rows of a
 * prefill chunk.
 *
 * The same Eq. 7 selection as nosa_select_blocks (same passages), with the
 * chunk treated as one query group: the G query heads of every row are
 * summed, as the G heads of one row are.  With c = pos[b][0] / 64 (the first
 * row's window; the variant is meant for chunks inside one block, as the
 * rows at the end of a prompt):
 *   qsum      = sum over rows r and the G heads of KV head h (fp32);
 *   sigma_s, score_j, Gamma_q, Gamma_e as in nosa_select_blocks over j < c;
 *   sel[b][r][h][..] = Gamma_q U Gamma_e ascending for every row r, the rest
 *   -1; n_sel[b][r][h] = its size.
 * Each row still attends its own window block in nosa_sparse_chunk_attn.
 * Arguments, layouts and workspace as nosa_select_blocks.
 * Errors: as nosa_select_blocks, and -2 unless the dtype is bf16 and G is
 * 1, 2, 4 or 8.
 */
int nosa_select_blocks_shared(const nosa_dims* dims, const void* q, int32_t n_query,
                              const int32_t* pos, const void* k_comp, const float* e_blk,
                              int32_t kq, int32_t ke, int32_t* sel, int32_t* n_sel, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * nosa_fetch_blocks -- keep the selected blocks in a fixed HBM block pool.
 *
 * Defined by the montaan summary ("System Optimization (NOSI)" item 2: KV in
 * block-sized units on GPU and CPU, only blocks unused in the current step
 * are swapped out; item 3: the host-to-device transfer reads host memory
 * directly through unified virtual addressing) and the gist.science summary
 * ("2. Système : NOSI": set differences drive block swapping; the wmrh.cn
 * post: only the window and the Top-K blocks stay on the GPU).
 * Per (b, h), with S = sel[b][h][0 .. n_sel-1] (one query row):
 *   1. if insert_block[b] = j >= 0 and j is not resident, j (the block the
 *      window just completed, held at insert_src) takes a slot first, with
 *      last_use = step - 1;
 *   2. the misses M = S minus the resident blocks, ascending, each take the
 *      lowest free slot, else the slot of the resident block not in S with
 *      the smallest (last_use, block id);
 *   3. last_use = step for every block of S; phys[i] = slot of S[i];
 *   4. the missing blocks are copied host -> pool by a gather kernel that
 *      reads the pinned host cache directly (zero-copy), and the inserted
 *      block is copied insert_src -> pool.
 * Table updates (1-3) run in one wavefront per (b, h); the copies (4) run as
 * a second kernel on the same stream (normally a side stream).
 *
 *   host_kv        pinned host [B][Hkv][NB][block]            (read)
 *   pool           device [B][Hkv][pool_slots][block]         (written)
 *   pool_slots     P, with kq + ke < P <= 1024
 *   block_table    device int32 [B][Hkv][NB]: slot or -1     (read/written)
 *   slot_block     device int32 [B][Hkv][P]: block or -1     (read/written)
 *   slot_last_use  device int32 [B][Hkv][P]                   (read/written)
 *                  (a fresh pool: block_table and slot_block all -1)
 *   step           the decode step t (host int)
 *   sel, n_sel     device, as written by nosa_select_blocks with n_query = 1;
 *                  k_cap = kq + ke <= 64 is the row length of sel; entries
 *                  outside [0, NB) are skipped
 *   insert_block   device int32 [B] or NULL (no insertion)
 *   insert_src     device [B][Hkv][block] or NULL (required with insert_block)
 *   phys           device int32 [B][Hkv][k_cap]: slot of each sel entry, -1
 *                  for skipped or padding entries                  (written)
 *   miss_list      device int32 [B][Hkv][k_cap + 1][2]: (block, slot) of each
 *                  miss in ascending block order; entry k_cap holds the
 *                  inserted block (or -1, -1)                      (written)
 *   n_miss         device int32 [B][Hkv]                             (written)
 */
int nosa_fetch_blocks(const nosa_dims* dims, const void* host_kv, void* pool,
                      int32_t pool_slots, int32_t* block_table, int32_t* slot_block,
                      int32_t* slot_last_use, int32_t step, const int32_t* sel,
                      const int32_t* n_sel, int32_t k_cap, const int32_t* insert_block,
                      const void* insert_src, int32_t* phys, int32_t* miss_list,
                      int32_t* n_miss, void* stream);

/*
 * nosa_update_pool, nosa_gather_blocks -- the two phases of
 * nosa_fetch_blocks as separate calls, so that work that needs only the
 * updated tables (the attention over the blocks already resident, see
 * nosa_sparse_decode_attn_pool) can run while the gather copies the misses.
 * nosa_update_pool runs steps 1-3 (tables, phys, miss list); nosa_gather_blocks
 * runs step 4 from the miss list, on any stream ordered after the update.
 * Arguments and errors as for nosa_fetch_blocks; the pair has exactly its
 * effect.  insert_src goes to the gather and is required there whenever the
 * update was given insert_block (else the inserted slot is not filled).
 */
int nosa_update_pool(const nosa_dims* dims, int32_t pool_slots, int32_t* block_table,
                     int32_t* slot_block, int32_t* slot_last_use, int32_t step, const int32_t* sel,
                     const int32_t* n_sel, int32_t k_cap, const int32_t* insert_block, int32_t* phys,
                     int32_t* miss_list, int32_t* n_miss, void* stream);
int nosa_gather_blocks(const nosa_dims* dims, const void* host_kv, void* pool, int32_t pool_slots,
                       int32_t k_cap, const void* insert_src, const int32_t* miss_list,
                       const int32_t* n_miss, void* stream);

/*
 * nosa_select_update_pool -- nosa_select_blocks (one query row per batch
 * entry) and nosa_update_pool in one launch.
 *
 * The selection (montaan summary, "Key Design Components" item 4, Eq. 7) and
 * the set difference against the pool (montaan, "System Optimization (NOSI)"
 * item 2; gist.science, "2. Système : NOSI") run back to back on the critical
 * path of an offloaded step: the workgroup that completes a (b, h)
 * selection updates that unit's pool from the set it has just written, so
 * the gather (nosa_gather_blocks, normally on a side stream) can follow
 * directly.  The effect is exactly that of
 *   nosa_select_blocks(dims, q, 1, pos, k_comp, e_blk, kq, ke, sel, n_sel, ws, ws_bytes, stream);
 *   nosa_update_pool(dims, pool_slots, block_table, slot_block, slot_last_use, step,
 *                    sel, n_sel, kq + ke, insert_block, phys, miss_list, n_miss, stream);
 * with every argument as documented there (sel and n_sel written, then
 * read).  kq + ke <= 64 (the pool's limit).  Errors: those of both calls,
 * checked before anything is launched.
 */
int nosa_select_update_pool(const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                            const float* e_blk, int32_t kq, int32_t ke, int32_t* sel, int32_t* n_sel,
                            void* ws, size_t ws_bytes, int32_t pool_slots, int32_t* block_table,
                            int32_t* slot_block, int32_t* slot_last_use, int32_t step,
                            const int32_t* insert_block, int32_t* phys, int32_t* miss_list,
                            int32_t* n_miss, void* stream);

/*
 * nosa_sparse_decode_attn -- exact attention over the selected blocks.
 *
 * Defined by the wmrh.cn NOSA-1B post ("工程实现亮点": two-stage attention,
 * the compressed KV picks the Top-K blocks, then exact attention on them;
 * "NOSA-1B 是什么": the current window and the Top-K blocks are kept).
 * For query head g of KV head h (g in 0..G-1, query head index h*G + g):
 *   T = tokens of the blocks phys[b][h][0 .. n_sel-1] plus the window
 *       tokens 64c .. p (p = pos[b], c = p / 64);
 *   out[b][h*G+g] = sum_{i in T} softmax_i(scale * q . K_i) V_i,
 * accumulated in fp32 (split over the blocks, merged with the usual
 * max/sum rescaling), stored once in the cache dtype (nearest-even).
 *
 *   q          device [B][Hq][D], cache dtype
 *   blocks     device base of the blocks phys refers to:
 *              [B][Hkv][blocks_per_head][block] (the full cache with phys =
 *              sel, or the HBM pool with phys from nosa_fetch_blocks)
 *   phys, n_sel  device int32 [B][Hkv][k_cap], [B][Hkv] (k_cap <= 512);
 *              entries outside [0, blocks_per_head) are skipped
 *   window_kv  device; the window block of (b, h) starts at element
 *              (b*Hkv + h) * window_head_stride + c * window_block_stride
 *              (cache: strides NB*block and block; a separate window buffer
 *              [B][Hkv][block]: strides block and 0)
 *   pos        device int32 [B]; entries outside [0, NB*64) give zeros
 *   scale      softmax scale (1/sqrt(D) for standard attention)
 *   out        device [B][Hq][D], cache dtype                    (written)
 *   ws         device workspace of at least
 *              nosa_workspace_size(dims, NOSA_OP_ATTN, 1, k_cap, 0) bytes,
 *              zero-filled once before its first use; every call leaves it
 *              ready for the next one.
 */
int nosa_sparse_decode_attn(const nosa_dims* dims, const void* q, const void* blocks,
                            int32_t blocks_per_head, const int32_t* phys,
                            const int32_t* n_sel, int32_t k_cap, const void* window_kv,
                            int64_t window_head_stride, int64_t window_block_stride,
                            const int32_t* pos, float scale, void* out, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * nosa_sparse_decode_attn_bias -- nosa_sparse_decode_attn over the resident
 * cache with each token's eviction logit added to its attention logit, a
 * variant kept for comparison (the path itself adds no bias, so that top-k
 * over every block is dense causal attention).
 *
 * The gist.science summary ("1. Algorithme : NOSA", ED-DMA) defers the
 * eviction head's exponential to the attention step; read as an additive
 * logit:
 *   out[b][h*G+g] = sum_{i in T} softmax_i(scale * q . K_i + L[b][h][i]) V_i
 * with T as in nosa_sparse_decode_attn and L = evict_logits (natural-log
 * units, the same for every query head of the KV head).
 *
 *   q, pos, scale, out, ws   as nosa_sparse_decode_attn
 *   kv            device cache [B][Hkv][NB][block]; the window is block
 *                 pos/64 of the cache
 *   sel, n_sel    device int32 [B][Hkv][k_cap], [B][Hkv] (k_cap <= 512), as
 *                 nosa_select_blocks writes them; entries outside [0, NB)
 *                 are skipped
 *   evict_logits  device fp32 [B][Hkv][NB*64], the logits nosa_pool_keys
 *                 pools
 * Errors as nosa_sparse_decode_attn.
 */
int nosa_sparse_decode_attn_bias(const nosa_dims* dims, const void* q, const void* kv, const int32_t* sel,
                                 const int32_t* n_sel, int32_t k_cap, const int32_t* pos, float scale,
                                 const float* evict_logits, void* out, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * nosa_sparse_decode_attn_pool -- nosa_sparse_decode_attn over the HBM pool
 * of an offload step, in two parts around the fetch's gather.  Same result
 * and arguments (blocks = the pool, blocks_per_head = pool_slots, phys from
 * nosa_update_pool), plus that call's miss_list and n_miss:
 *   part 0  attends the selected blocks whose slots this step's gather does
 *           not write (the hits) and the window; it writes partials to ws
 *           only.  Needs nosa_update_pool done, not the gather: run it
 *           while the gather runs.
 *   part 1  attends the slots the gather filled (the misses, and the block
 *           the window completed when it is selected), then merges with
 *           part 0's partials into out.  Needs part 0 and the gather done.
 * Communication is the bottleneck of offloaded decoding (montaan summary,
 * "Empirical Results and Analysis"; gist.science "Résultats
 * Expérimentaux"), so the attention over the hits is moved off its path.
 *   part       0 or 1
 *   ws         as for nosa_sparse_decode_attn, shared by the two parts of a
 *              step; part 1 leaves it ready for the next step.
 */
int nosa_sparse_decode_attn_pool(const nosa_dims* dims, const void* q, const void* pool,
                                 int32_t pool_slots, const int32_t* phys, const int32_t* n_sel,
                                 int32_t k_cap, const int32_t* miss_list, const int32_t* n_miss,
                                 const void* window_kv, int64_t window_head_stride,
                                 int64_t window_block_stride, const int32_t* pos, float scale,
                                 int32_t part, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * nosa_sparse_decode_attn_fetch -- the gather and the attention of an
 * offload step in one launch.
 *
 * NOSI moves the missing blocks with a zero-copy read of host memory
 * through unified virtual addressing (montaan summary, "System Optimization
 * (NOSI)" item 3).  Here the read feeds the attention directly: a fetched
 * block comes from the host cache into the registers of the wavefront that
 * attends it, which also writes it to its pool slot, while the other
 * wavefronts attend the blocks already resident.  The effect is exactly
 * that of
 *   nosa_gather_blocks(dims, host_kv, pool, pool_slots, k_cap, insert_src, miss_list, n_miss, stream);
 *   nosa_sparse_decode_attn(dims, q, pool, pool_slots, phys, n_sel, k_cap, window_kv,
 *                           window_head_stride, window_block_stride, pos, scale, out, ws, ws_bytes, stream);
 * on one stream, after nosa_update_pool (or nosa_select_update_pool) of the
 * step, with every argument as documented there; k_cap <= 64.  The pool
 * slots this step fills are written, the others only read.
 * Errors as those two calls (host_kv must not be NULL).
 */
int nosa_sparse_decode_attn_fetch(const nosa_dims* dims, const void* q, const void* host_kv, void* pool,
                                  int32_t pool_slots, const int32_t* phys, const int32_t* n_sel,
                                  int32_t k_cap, const int32_t* miss_list, const int32_t* n_miss,
                                  const void* insert_src, const void* window_kv,
                                  int64_t window_head_stride, int64_t window_block_stride,
                                  const int32_t* pos, float scale, void* out, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * nosa_sparse_chunk_attn -- exact attention for n_query rows of one batch
 * entry (a prefill chunk), each row over its own selection and its own
 * causal window, from the resident cache.
 *
 * Defined by the same passages as nosa_sparse_decode_attn, per query row:
 * row r of batch entry b at position p = pos[b][r] attends the blocks
 * sel[b][r][h][0 .. n_sel[b][r][h]-1] (as written by nosa_select_blocks with
 * the same n_query) plus tokens 64c .. p of block c = p / 64, read from kv.
 *
 *   q        device [B][n_query][Hq][D], cache dtype
 *   kv       device cache [B][Hkv][NB][block]
 *   sel, n_sel  device int32 [B][n_query][Hkv][k_cap], [B][n_query][Hkv]
 *            (k_cap <= 512); entries outside [0, NB) are skipped.  A row's
 *            entries are distinct blocks before its window block, as
 *            nosa_select_blocks writes them (a repeated entry, or the
 *            window block itself, is not defined).
 *   pos      device int32 [B][n_query]; rows outside [0, NB*64) give zeros
 *   out      device [B][n_query][Hq][D], cache dtype                (written)
 *   ws       device workspace of at least
 *            nosa_workspace_size(dims, NOSA_OP_ATTN, n_query, k_cap, 0) bytes,
 *            zero-filled once before its first use.
 * Errors as nosa_sparse_decode_attn; also -1 for n_query < 1 and -2 when
 * B * n_query * Hkv exceeds 65535.
 */
int nosa_sparse_chunk_attn(const nosa_dims* dims, const void* q, int32_t n_query, const void* kv,
                           const int32_t* sel, const int32_t* n_sel, int32_t k_cap, const int32_t* pos,
                           float scale, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * nosa_decode_step -- one decode step of a resident cache in one launch:
 * nosa_select_blocks (n_query = 1) followed by nosa_sparse_decode_attn over
 * the cache, with the same results.
 *
 * Follows from the same passages.  The query-agnostic set Gamma_e depends
 * only on the block eviction scores, which do not change once a block is
 * complete (gist.science summary, "1. Algorithme : NOSA": the eviction head
 * scores KV pairs independently of the query), so the attention over Gamma_e
 * and the window runs while the compressed-key scan for Gamma_q is still in
 * flight; only the blocks of Gamma_q outside Gamma_e wait for the scan.
 *
 *   q, pos, k_comp, e_blk, kq, ke   as for nosa_select_blocks (n_query = 1;
 *                    pos is [B]); kq + ke <= 256; at most 8 query heads per
 *                    KV head
 *   kv       device [B][Hkv][NB][block]: the cache, read in place (the
 *            window is block pos/64 of the cache)
 *   scale    softmax scale
 *   sel, n_sel  device [B][Hkv][kq+ke], [B][Hkv]: the selected blocks
 *            (ascending, -1 padded), as nosa_select_blocks writes them
 *   out      device [B][Hq][D], cache dtype                      (written)
 *   ws       device workspace of nosa_workspace_size(dims, NOSA_OP_STEP,
 *            1, kq, ke) bytes, zero-filled once before its first use (and
 *            again before it is used with other dims, kq or ke).  It keeps
 *            an arrival counter per (b, h) and Gamma_e per (b, h) between
 *            calls, keyed by the e_blk address and the window block: the
 *            eviction scores at that address must not change for blocks
 *            before the window between calls with the same window block
 *            (they never do in decoding, where a block's score is fixed once
 *            it is complete; zero-fill the workspace again after changing
 *            them).  Calls sharing a workspace must not overlap.
 * The kernel's workgroups hand partial results to each other through the
 * workspace; every such wait is bounded (about 0.3 s).  A wait that hits its
 * bound -- only possible if the device did not run the workgroups of one
 * launch concurrently -- is counted in the workspace and turns the outputs
 * it feeds into NaN; nosa_step_timeouts reads the count.
 */
int nosa_decode_step(const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                     const float* e_blk, int32_t kq, int32_t ke, const void* kv, float scale,
                     int32_t* sel, int32_t* n_sel, void* out, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * nosa_decode_step_static -- nosa_decode_step with no workspace argument and
 * no allocation: for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments (minus ws, ws_bytes), results and errors as
 * nosa_decode_step.  The workspace is the library's own: one 16 MiB device
 * array per device, held until the process ends, zero-filled on the first
 * call on a device and whenever the geometry (dims, kq, ke) differs from the
 * previous call's on that device.  Every call on a device shares it and it
 * keeps the last call's contents, so calls that overlap on one device (other
 * streams, other threads) race; calls in stream order do not.  Gamma_e is
 * cached in it keyed by the e_blk address and the window block, as in
 * nosa_decode_step.  A geometry whose workspace (nosa_workspace_size with
 * NOSA_OP_STEP) exceeds 16 MiB is rejected with -4.  The call allocates and
 * frees nothing; the first call on a device looks up the array's address.
 * Under graph capture the geometry check (and the clear it may launch) runs
 * when a call is captured, not when the graph is replayed: make one call of
 * the geometry before capturing, so that the graph holds the step launches
 * only, and after calls of another geometry on the device make one call of
 * the graph's geometry outside the graph before replaying it.
 */
int nosa_decode_step_static(const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                            const float* e_blk, int32_t kq, int32_t ke, const void* kv, float scale,
                            int32_t* sel, int32_t* n_sel, void* out, void* stream);

/*
 * nosa_step_timeouts -- the number of bounded hand-off waits of
 * nosa_decode_step that hit their bound so far in workspace ws (0 when every
 * launch ran as it should).
 *
 *   dims, kq, ke  as given to nosa_decode_step with this workspace
 *   ws            the step workspace (device); NULL: this device's static
 *                 workspace of nosa_decode_step_static
 *   out           device memory, or pinned host memory the device can write
 *                 (hipHostMalloc), receiving one int32            (written)
 * Enqueued on `stream` after the steps to be checked; the caller reads out
 * once the stream has reached it.  Errors: -1 for a NULL out, negative
 * budgets, or ws = NULL before nosa_decode_step_static ran on this device.
 */
int nosa_step_timeouts(const nosa_dims* dims, int32_t kq, int32_t ke, const void* ws, int32_t* out,
                       void* stream);

/*
 * nosa_debug_expire_step_waits -- a test hook for the one-launch step's
 * failure handling, for test suites only.  While on (on != 0), every launch
 * of nosa_decode_step and nosa_decode_step_static that follows treats the
 * query-aware workers' score words as not yet written and bounds that wait
 * at 64 polls, so each of those waits expires: the launch counts them
 * (nosa_step_timeouts) and writes NaN for every output (with kq > 0; kq = 0
 * has no such wait), and every kernel still runs to its end.  on = 0 restores normal launches.  Process-wide,
 * affects launches issued after the call; off by default; returns 0.
 */
int nosa_debug_expire_step_waits(int32_t on);

/* Workspace bytes needed by op (NOSA_OP_SELECT, NOSA_OP_ATTN or NOSA_OP_STEP); 0 on bad input. */
size_t nosa_workspace_size(const nosa_dims* dims, int32_t op, int32_t n_query, int32_t kq,
                           int32_t ke);

/* Static text of a status code. */
const char* nosa_status_str(int32_t status);

/* Text of the last failure on the calling thread ("" if none). */
const char* nosa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NOSA_H */
