/*
 * flexattn.h - C ABI of the fused, tiled attention forward for AMD MI355X (gfx950).
 *
 * What it computes. For every batch b, query head h and query position q:
 *
 *     s[j]   = scale * dot(Q[b,h,q,:], K[b,kvh,j,:])          kvh = h / (H / Hkv)
 *     s'[j]  = score_mod(s[j], b, h, q, j)
 *     O[b,h,q,:] = sum_{j : mask_mod(b,h,q,j)} softmax_j(s') V[b,kvh,j,:]
 *     LSE[b,h,q] = log sum_{j : mask_mod(b,h,q,j)} exp(s'[j])      (natural log)
 *
 * A row that admits no key gets O = 0 and LSE = -inf.
 *
 * This is softmax attention comparing every query with every key (Neuron FA4
 * explainer, "What Is Attention, and Why Is It Expensive?"), computed tile by
 * tile in on-chip memory so that the score matrix is never written to HBM and
 * with no approximation (same page, "Enter Tri Dao and FlashAttention";
 * NextVector FlexAttention article, "Executive Key Takeaways"). The score and
 * mask modifications are the FlexAttention-style variants the pages list
 * (sliding window, document packing, ALiBi, soft-capping: Neuron FA4
 * explainer, "PyTorch Gets the Upgrade Too"; NextVector article, "What
 * Happened?"), selected here by enum and compiled in, rather than generated
 * at run time (PyTorch FlexAttention FA4-backend post).
 *
 * Conventions for every call below:
 *   - Tensors are caller-owned device memory (e.g. allocated by PyTorch),
 *     contiguous, row-major in the shapes given. The library allocates
 *     nothing, keeps no pointer after a call returns and has no mutable
 *     global state; calls are reentrant.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call returns a negative FLEXATTN_ERR_* code and touches no memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising. A fault inside a kernel
 *     surfaces at the caller's next synchronisation on that stream.
 */
#ifndef FLEXATTN_H
#define FLEXATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLEXATTN_VERSION 4

/* Block-mask tiles: FLEXATTN_QTILE query rows (two halves of FLEXATTN_TILE
 * rows) by FLEXATTN_TILE keys. */
#define FLEXATTN_TILE 128
#define FLEXATTN_QTILE 256

/* Status codes: 0 on success, negative on failure. */
enum flexattn_status {
  FLEXATTN_OK = 0,
  FLEXATTN_ERR_NULLPTR = -1,     /* a required pointer is NULL                         */
  FLEXATTN_ERR_SHAPE = -2,       /* B, H, Hkv, Sq, Skv < 1, or H % Hkv != 0            */
  FLEXATTN_ERR_UNSUPPORTED = -3, /* D not 64/128/256, unknown dtype, mask or mod kind  */
  FLEXATTN_ERR_ALIGN = -4,       /* Q/K/V/O not 16-byte or LSE/params not 4-byte aligned */
  FLEXATTN_ERR_BLOCKMASK = -5,   /* block mask does not match the call                 */
  FLEXATTN_ERR_OVERFLOW = -6,    /* sizes exceed the 32-bit index range (also: one
                                    (batch, head) slice must stay below 2^31 bytes)    */
  FLEXATTN_ERR_HIP = -7,         /* a HIP call failed; see flexattn_last_error()       */
  FLEXATTN_ERR_ARG = -8,         /* bad scalar argument (scale, window, softcap, size,
                                    stride; overlapping gradient layouts)              */
  FLEXATTN_ERR_SCRATCH = -9      /* flexattn_decode_static: the call's split results
                                    exceed FLEXATTN_STATIC_SCRATCH_BYTES              */
};

/* Element type of Q, K, V and O. LSE is always float32. FP32 inputs are
 * rounded to bf16 (round-to-nearest-even) when loaded, since both products
 * run on bf16 matrix cores with float32 accumulation; O is stored as float32. */
enum flexattn_dtype { FLEXATTN_BF16 = 0, FLEXATTN_FP32 = 1 };

/* Positions. Key j sits at position k_idx = j; query row i sits at position
 * q_idx = i + params->q_offset (0 by default: rows and keys start together).
 * Masks, score mods and document labels see positions, so decoding or a
 * prefill chunk that follows Skv - Sq cached keys passes q_offset = Skv - Sq.
 *
 * mask_mod kinds: bit flags, AND-composed; 0 = every key admitted.
 *   CAUSAL   : q_idx >= k_idx
 *   WINDOW   : q_idx - k_idx < params->window       (combine with CAUSAL for a
 *                                                      causal sliding window)
 *   DOCUMENT : doc[b][q_idx] == doc[b][k_idx]        (document packing)
 *   PREFIX   : with CAUSAL only: the causal part becomes
 *              q_idx >= k_idx || k_idx < params->prefix (prefix-LM: the prefix
 *              is seen by every query; WINDOW and DOCUMENT still apply)
 * The pages name prefix masking among FlexAttention's variants without
 * defining it (PyTorch 2.5 / FlexAttention article, overview and "What
 * Happened?"); the prefix-LM reading above is this library's.              */
enum flexattn_mask_kind {
  FLEXATTN_MASK_NONE = 0,
  FLEXATTN_MASK_CAUSAL = 1,
  FLEXATTN_MASK_WINDOW = 2,
  FLEXATTN_MASK_DOCUMENT = 4,
  FLEXATTN_MASK_PREFIX = 8
};

/* score_mod kinds, applied to the scaled score s = scale * q.k:
 *   ALIBI   : s + alibi_slopes[h] * (k_idx - q_idx)      (positions, as above)
 *   SOFTCAP : softcap * tanh(s / softcap)
 *   RELBIAS : s + rel_bias[h][clip(k_idx - q_idx, -R, R) + R], R = rel_max
 *             (relative position bias: a per-head table over the clipped
 *             relative position; the pages name relative position encodings
 *             among FlexAttention's variants, PyTorch 2.5 / FlexAttention
 *             article, overview)                                                */
enum flexattn_mod_kind {
  FLEXATTN_MOD_NONE = 0,
  FLEXATTN_MOD_ALIBI = 1,
  FLEXATTN_MOD_SOFTCAP = 2,
  FLEXATTN_MOD_RELBIAS = 3
};

/* Largest clip distance R of a relative-bias table (tables are staged in LDS). */
#define FLEXATTN_REL_MAX 1023

/* Parameters of the variants. Host struct, read during the call only.
 * A NULL params pointer means: dtype BF16, no window, no documents, no mods,
 * q_offset 0. */
typedef struct flexattn_params {
  int dtype;                 /* enum flexattn_dtype                                   */
  int window;                /* > 0 when the mask has FLEXATTN_MASK_WINDOW            */
  float softcap;             /* > 0 when mod_kind is FLEXATTN_MOD_SOFTCAP             */
  const float* alibi_slopes; /* device float32 [H] when mod_kind is FLEXATTN_MOD_ALIBI */
  const int* doc_ids;        /* device int32 [B][doc_stride] document label per position,
                                when the mask has FLEXATTN_MASK_DOCUMENT               */
  int doc_stride;            /* elements per batch row of doc_ids,
                                >= max(Sq + q_offset, Skv), <= INT_MAX / 4 and
                                B * doc_stride <= INT_MAX (else ERR_OVERFLOW)          */
  int q_offset;              /* >= 0: position of query row 0 (see "Positions")       */
  int prefix;                /* >= 0 when the mask has FLEXATTN_MASK_PREFIX           */
  const float* rel_bias;     /* device float32 [H][2 * rel_max + 1], 16-byte aligned,
                                when mod_kind is FLEXATTN_MOD_RELBIAS                  */
  int rel_max;               /* R in [0, FLEXATTN_REL_MAX] for FLEXATTN_MOD_RELBIAS   */
  /* Layout of q, k, v and out: element strides {batch, head, row}; the last
   * (D) dimension is always contiguous. All three zero (the default) means the
   * contiguous [B][H][S][D] layout; e.g. a [B][S][H][D] buffer viewed as
   * [B][H][S][D] has strides {S*H*D, D, H*D}. Strides are >= 0, a row stride
   * is >= D, and each stride times the element size is a multiple of 16
   * bytes (else FLEXATTN_ERR_ALIGN). LSE is always contiguous [B][H][Sq].
   * flexattn_bwd applies the same strides to the gradients: dq takes
   * q_stride, dk k_stride, dv v_stride and dout o_stride.
   * Every layout that is written must not overlap: out in every call, and in
   * flexattn_bwd also q, k and v (whose strides the gradients take). "Not
   * overlapping" is tested as: ordered by stride, each dimension of extent
   * > 1 steps over the span of those below it (so no stride 0 over a
   * dimension longer than 1); else FLEXATTN_ERR_ARG. The forward only reads
   * q, k and v, so it accepts overlapping (e.g. broadcast) inputs.          */
  long long q_stride[3], k_stride[3], v_stride[3], o_stride[3];
} flexattn_params;

/* Block mask: for every query tile of FLEXATTN_QTILE rows, the ascending list
 * of key tiles of FLEXATTN_TILE keys that hold at least one admitted pair for
 * either half of the query tile (rows 0-127 = half 0, rows 128-255 = half 1).
 * Each entry is
 *     (kv_tile << 4) | full1 << 3 | any1 << 2 | full0 << 1 | any0
 * where any_h says the half has an admitted pair in the tile and full_h that
 * every pair of the half is in range and admitted (the kernel then skips the
 * per-element mask). Tiles empty for both halves are absent and never
 * computed; a half that is empty in a listed tile skips it.
 * The lists depend on the batch only through DOCUMENT masks (num_b = B then,
 * else num_b = 1 and row 0 serves every batch); no mask depends on the head.
 * Filled in by flexattn_build_block_mask; the arrays live in the caller's
 * buffer. */
typedef struct flexattn_block_mask {
  int tile_q, tile_k;   /* FLEXATTN_QTILE, FLEXATTN_TILE                         */
  int nq, nk;           /* ceil(Sq / tile_q), ceil(Skv / tile_k)                  */
  int num_b;            /* 1 or B                                                */
  int mask_kind;        /* the mask_kind it was built for                        */
  int Sq, Skv;          /* the sizes it was built for                            */
  const int* kv_count;  /* device int32 [num_b][nq]: entries in each list        */
  const int* kv_list;   /* device int32 [num_b][nq][nk]: entries as above,
                           ascending; entries past kv_count are unspecified      */
  int window, q_offset, prefix;  /* the params it was built for (0 where the mask
                                    kind does not use them)                      */
} flexattn_block_mask;

/* Library version (FLEXATTN_VERSION of the build). */
int flexattn_version(void);

/* Static text for a status code. Never NULL. */
const char* flexattn_strerror(int status);

/* Detail text of the last FLEXATTN_ERR_HIP returned on this thread ("" if none). */
const char* flexattn_last_error(void);

/* Dispatch log: when the environment variable FLEXATTN_LOG is set to anything
 * but "" or "0" (read once per process), flexattn_fwd, flexattn_decode,
 * flexattn_decode_static, flexattn_bwd and flexattn_build_block_mask each
 * print one line on stderr as they return: "[flexattn] <entry>(<arguments>)
 * -> <kernels launched, with template arguments and grid, or 'no launch'>
 * -> <status> (<flexattn_strerror text>)". */

/* Bytes of device memory flexattn_build_block_mask needs for these sizes
 * (int32 counts and lists). Returns 0 for invalid sizes or mask kinds. */
size_t flexattn_block_mask_bytes(int B, int Sq, int Skv, int mask_kind);

/* Classify every (query half-tile, key tile) pair of the mask as full,
 * partial or empty and write the per-query-tile key-tile lists into `buf` (device memory
 * of at least flexattn_block_mask_bytes(B, Sq, Skv, mask_kind) bytes, 4-byte
 * aligned). `params` supplies window, doc_ids, q_offset and prefix as for
 * flexattn_fwd (may be NULL when the mask needs none of them). On success
 * fills *out (which records those parameters: a call whose params differ
 * where the mask uses them gets FLEXATTN_ERR_BLOCKMASK), whose pointers
 * point into buf, and enqueues the build on `stream`. A half is marked full
 * exactly when every pair in it is in range and admitted, and absent only when
 * no pair in it is admitted. Without DOCUMENT masks the classes are exact;
 * with them, a half whose document labels overlap those of the key tile
 * without all being one label may be listed as partial although no pair in
 * it is admitted (the forward kernel's per-element mask then admits nothing
 * there, so results do not change). */
int flexattn_build_block_mask(int mask_kind, const flexattn_params* params, int B, int Sq, int Skv,
                              void* buf, size_t bytes, flexattn_block_mask* out, void* stream);

/* Attention forward.
 *   q     : device [B][H][Sq][D]    dtype of params (bf16 or float32)
 *   k, v  : device [B][Hkv][Skv][D] same dtype
 *   out   : device [B][H][Sq][D]    same dtype; every element is written
 *   lse   : device float32 [B][H][Sq], or NULL to skip it; every element is written
 *   D     : 64, 128 or 256 (256: bf16, Skv <= 2048 * FLEXATTN_TILE); scale:
 *           finite and > 0 (1/sqrt(D) is the usual choice)
 *   mask_kind, mod_kind, params: the variant (see above)
 *   block_mask: from flexattn_build_block_mask for the same mask_kind, sizes
 *           and params, or NULL to visit every key tile with the per-element
 *           mask (correct for any mask, slower). With mask_kind 0 (no mask)
 *           NULL costs nothing: every key tile inside Skv is then taken as
 *           full, the last one partial when Skv is not a multiple of
 *           FLEXATTN_TILE, as the built mask would classify them. Results are
 *           bitwise equal either way.
 * Query head h reads key/value head h / (H / Hkv). */
int flexattn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                 int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                 const flexattn_params* params, const flexattn_block_mask* block_mask,
                 void* stream);

/* Split-KV attention forward: what flexattn_fwd computes, with each item's
 * key tiles split over `splits` workgroups (1 <= splits <= 64) whose
 * normalised partial results are merged as O = sum_s exp(LSE_s - LSE) O_s,
 * LSE = log sum_s exp(LSE_s) by a second kernel on the same stream. Two
 * organisations, chosen by the shape:
 *   rep * Sq <= 256 (rep = H / Hkv; decoding, Sq = 1 with q_offset = Skv - 1,
 *     and short prefill chunks): the rep query heads of a key/value head
 *     share a workgroup as rep * Sq packed rows, so each K/V element is read
 *     once; with FLEXATTN_MOD_RELBIAS the group's tables must fit together:
 *     rep * (2 * rel_max + 1) <= 2 * FLEXATTN_REL_MAX + 2;
 *   otherwise: flexattn_fwd's 256-row query tiles, each tile's key list cut
 *     into `splits` contiguous parts, for grids too small to fill the chip
 *     (few heads, long causal rows).
 * Faster inference and longer contexts are among the uses the pages give the
 * method (Neuron FA4 explainer, "Why This Matters for Everyone"); splitting
 * the keys is how one query row, or a few heads, fill the chip, and the
 * merge is the log-sum-exp identity of the forward's own LSE output. bf16
 * only; every variant and layout of flexattn_fwd;
 * block_mask as there (built for these Sq, Skv); B * H * ceil(Sq / 256) *
 * splits <= INT_MAX (else FLEXATTN_ERR_OVERFLOW).
 *   workspace : device memory of flexattn_decode_workspace_bytes(...) bytes,
 *               16-byte aligned, caller-owned scratch (contents afterwards
 *               unspecified); may be NULL when splits == 1
 * Results equal flexattn_fwd's up to float32 rounding in the merge. */
size_t flexattn_decode_workspace_bytes(int B, int H, int Hkv, int Sq, int D, int splits);

/* A split count for packed decoding (rep * Sq <= 256): a decode-mode
 * workgroup fills a CU, so B * Hkv * splits workgroups run in
 * ceil(B * Hkv * splits / 256) rounds, each taking about 2 * tiles / splits
 * + 3 stage times (tiles = ceil(Skv / 128), two stages per tile, ~3 stages
 * of start and drain per workgroup). The count minimises that product (the
 * fewest splits among equals), at most 64 and leaving each split at least
 * 4 key tiles. */
int flexattn_decode_splits(int B, int Hkv, int Skv);

/* A split count for flexattn_decode in either organisation: the packed rule
 * above, else 1 when B * H * ceil(Sq / 256) already gives ~2 workgroups per
 * CU, otherwise enough splits for that while each split of a whole key list
 * keeps at least 8 key tiles. Invalid sizes give 1. */
int flexattn_split_count(int B, int H, int Hkv, int Sq, int Skv);

int flexattn_decode(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                    int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                    const flexattn_params* params, const flexattn_block_mask* block_mask, int splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/* flexattn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as flexattn_decode (bitwise: the same kernels),
 * without the workspace: the split results go to a scratch array that the
 * library holds in device memory, FLEXATTN_STATIC_SCRATCH_BYTES per device,
 * from the first call on a device until the process ends. The call allocates
 * nothing.
 *   splits : 1..64; the split results take
 *            flexattn_decode_workspace_bytes(B, H, Hkv, Sq, D, splits) bytes
 *            of the scratch, and a call needing more than
 *            FLEXATTN_STATIC_SCRATCH_BYTES fails with FLEXATTN_ERR_SCRATCH
 *            (flexattn_last_error() gives the sizes) before any HIP call
 *   stream : must belong to the current device (else FLEXATTN_ERR_ARG); the
 *            first call on a device looks up that device's scratch address
 * Every call on one device shares that device's scratch, and the contents
 * last written stay until the next call overwrites them (nothing in it needs
 * to start at zero: every split writes all of its rows before the merge reads
 * them). Calls that overlap in time on one device (other streams, other host
 * threads) race on the scratch and give undefined results: order them. */
#define FLEXATTN_STATIC_SCRATCH_BYTES (64u << 20)
int flexattn_decode_static(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                           int H, int Hkv, int Sq, int Skv, int D, float scale, int mask_kind,
                           int mod_kind, const flexattn_params* params,
                           const flexattn_block_mask* block_mask, int splits, void* stream);

/* Attention backward: the gradients of L = sum(O * dout) with respect to q, k
 * and v, for O = flexattn_fwd(q, k, v, ...) with the same variant. The pages
 * name a backward pass used in training and a deterministic mode for it
 * (Neuron FA4 explainer, "FlashAttention-4: Built for Blackwell", backward-pass
 * fixes); the gradients follow from the definition above by differentiation.
 *   q, k, v    : as for flexattn_fwd; bf16 only (params->dtype = FLEXATTN_BF16),
 *                D = 64, 128 or 256, Skv <= 2048 * FLEXATTN_TILE (else
 *                FLEXATTN_ERR_UNSUPPORTED); layouts as given by params (see
 *                flexattn_params: each gradient takes its input's strides)
 *   out, lse   : the forward's O [B][H][Sq][D] bf16 and LSE [B][H][Sq] float32
 *   dout       : device [B][H][Sq][D] bf16, the gradient arriving at O
 *   dq         : device [B][H][Sq][D] bf16; every element is written
 *   dk, dv     : device [B][Hkv][Skv][D] bf16; every element is written (with
 *                grouped heads, the sum over the query heads of the group)
 *   delta      : device float32 [B][H][Sq], caller-owned scratch that the call
 *                overwrites with rowsum(dout * out); its contents afterwards
 *                are unspecified
 *   block_mask : as for flexattn_fwd, or NULL. dq visits its key tiles;
 *                dk/dv (D = 64, 128) under a document mask also read the
 *                lists to skip query rows that see none of a key tile and
 *                to treat fully admitted ones as full; other masks (and
 *                NULL) give dk/dv the query range from the causal and
 *                window parts. Results do not depend on whether it is given
 * Each gradient element is accumulated in a fixed order by one thread (no
 * atomics), so results are bitwise reproducible run to run. */
int flexattn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H,
                 int Hkv, int Sq, int Skv, int D, float scale, int mask_kind, int mod_kind,
                 const flexattn_params* params, const flexattn_block_mask* block_mask,
                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLEXATTN_H */
