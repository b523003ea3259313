// attn_fwd.hip - fused, tiled attention forward for gfx950 (MI355X, CDNA4).
//
// The method: keep the work of attention in on-chip memory instead of writing
// the score matrix to HBM and reading it back, with no approximation (Neuron FA4
// explainer, "Enter Tri Dao and FlashAttention"); run the softmax online, one key
// tile at a time, rescaling the running output when the running maximum grows
// (same page, "FlashAttention-4: Built for Blackwell", forward-pass fixes); split
// the work over query tiles, FlashAttention-2's improvement in how work is
// divided among parallel units (same page, "Enter Tri Dao and FlashAttention").
//
// Mapping to CDNA4:
//  * A workgroup owns one 128-row query tile of one (batch, head): 4 waves of 64
//    lanes, each wave 32 query rows. Grid ids are remapped so that the query
//    tiles of one (batch, key/value head) land on the same XCD and share its L2.
//  * Per 64-key stage each wave computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16 (fp32 accumulate). In the accumulator layout a
//    lane then holds 32 scores of ONE query row, so the row max needs one
//    permlane32 swap and the running sum stays lane-local until the epilogue.
//  * O^T += V^T P^T: the S^T accumulators, rounded to bf16, are already the
//    B operand (P^T) of the second MFMA; V is stored transposed in LDS with the
//    key order permuted to match, so each A-operand fetch is one 16-byte read.
//  * K and V^T stages are double-buffered in LDS; the next stage's global loads
//    are issued before the current stage's math and written to LDS after it.
//    All global reads are buffer loads whose range is one (batch, head) slice,
//    so rows past the end read as zero without any branch.
//  * Conditional rescaling (Neuron FA4 explainer, "FlashAttention-4: Built for
//    Blackwell", forward-pass fixes): the running max used as the exponent base
//    is raised only when some row of the wave grows by more than kRescaleLog2;
//    otherwise the stale base is kept, exponentials stay below 2^kRescaleLog2,
//    and O and the running sum are not touched. The final O / l and
//    LSE = base + log2(l) are the same quantities in exact arithmetic.
//  * LDS rows are padded by 16 bytes (K rows: D+8, V^T rows: 72 bf16). With
//    gfx950's 64 four-byte banks this makes the 16-byte fragment reads of both
//    products conflict-free, and the V^T stores conflict-free because the 16
//    lanes written together hold 16 different key groups of one column.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "launch.h"
#include "variants.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 waves
constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per pipeline stage
constexpr int kTile = 128;      // block-mask tile edge
constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

template <int D>
struct Geo {
  static constexpr int kStride = D + 8;            // bf16 per K row in LDS
  static constexpr int vStride = kBN + 8;          // bf16 per V^T row in LDS
  static constexpr int kElems = kBN * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int stage = kElems + vElems;    // bf16 per buffer
  static constexpr int kChunks = kBN * D / 8 / kThreads;  // 16B K chunks per thread
  static constexpr int vCols = kBN * D / (4 * kThreads);  // V columns per thread (4 rows each)
  static_assert(kChunks >= 1 && vCols >= 2 && (D / vCols) == 16, "tile geometry");
};

// 8 consecutive elements at element offset `eo`, as 4 packed bf16 pairs
// (fp32 sources rounded to nearest even).
template <bool F32>
__device__ inline u32x4 buf_load8(rsrc_t r, unsigned eo) {
  if constexpr (!F32) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, eo * 2u, 0, 0);
  } else {
    u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, eo * 4u, 0, 0);
    u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, eo * 4u + 16u, 0, 0);
    u32x4 o;
    o[0] = pack_bf16(__uint_as_float(a[0]), __uint_as_float(a[1]));
    o[1] = pack_bf16(__uint_as_float(a[2]), __uint_as_float(a[3]));
    o[2] = pack_bf16(__uint_as_float(b[0]), __uint_as_float(b[1]));
    o[3] = pack_bf16(__uint_as_float(b[2]), __uint_as_float(b[3]));
    return o;
  }
}

// N (4 or 8) consecutive elements as N/2 packed bf16 pairs.
template <bool F32, int N>
__device__ inline void buf_loadN(rsrc_t r, unsigned eo, unsigned (&dst)[N / 2]) {
  if constexpr (N == 8) {
    u32x4 v = buf_load8<F32>(r, eo);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = v[i];
  } else {
    static_assert(N == 4, "4 or 8 elements");
    if constexpr (!F32) {
      u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, eo * 2u, 0, 0);
      dst[0] = v[0];
      dst[1] = v[1];
    } else {
      u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, eo * 4u, 0, 0);
      dst[0] = pack_bf16(__uint_as_float(a[0]), __uint_as_float(a[1]));
      dst[1] = pack_bf16(__uint_as_float(a[2]), __uint_as_float(a[3]));
    }
  }
}

template <int D, int MOD, bool F32, bool DOCS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdLaunch p, const int* __restrict__ kv_count, const int* __restrict__ kv_list) {
  using G = Geo<D>;
  constexpr int DC = D / 16;          // 16-wide d chunks (QK^T k-steps)
  constexpr int DB = D / 32;          // 32-wide d blocks of O^T
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * G::stage];
  __shared__ float rtab[MOD == kModRelBias ? kRelCap : 1];   // this head's bias table

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;            // lane half

  // ---- workgroup -> (b, h, query tile), XCD-aware and heavy-tiles-first
  const int nq = (p.Sq + kBM - 1) / kBM;
  const int total = p.B * p.H * nq;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int wg = blockIdx.x;
  const int lin = (wg % kXcds) * per_xcd + wg / kXcds;
  if (lin >= total) return;
  const int qt = nq - 1 - (lin % nq);
  const int bh = lin / nq;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int kvh = h / (p.H / p.Hkv);

  const size_t q_head = (static_cast<size_t>(b) * p.H + h) * p.Sq;   // LSE rows

  constexpr unsigned esz = F32 ? 4u : 2u;
  // a (batch, head) slice spans rows 0 .. S - 1 (row strides in elements),
  // so rows past the end read as zero
  const char* qbase = static_cast<const char*>(p.q) + (b * p.q_sb + h * p.q_sh) * esz;
  const char* kbase = static_cast<const char*>(p.k) + (b * p.k_sb + kvh * p.k_sh) * esz;
  const char* vbase = static_cast<const char*>(p.v) + (b * p.v_sb + kvh * p.v_sh) * esz;
  const rsrc_t rq = make_rsrc(qbase, (static_cast<unsigned>(p.Sq - 1) * p.q_sr + D) * esz);
  const rsrc_t rk = make_rsrc(kbase, (static_cast<unsigned>(p.Skv - 1) * p.k_sr + D) * esz);
  const rsrc_t rv = make_rsrc(vbase, (static_cast<unsigned>(p.Skv - 1) * p.v_sr + D) * esz);

  // ---- this wave's 32 query rows; lane owns row q_row
  const int q_row = qt * kBM + wave * 32 + l32;
  const bool q_ok = q_row < p.Sq;

  // Q^T fragments (B operand): 8 consecutive d per lane half per 16-wide chunk;
  // rows past Sq read as zero
  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, buf_load8<F32>(rq, static_cast<unsigned>(q_row) * p.q_sr + c * 16 + g * 8));

  // ---- key-tile schedule
  const int bm_b = (kv_count && p.bm_num_b > 1) ? b : 0;
  // (kv_count / kv_list are separate __restrict__ arguments so that these
  // wave-uniform reads compile to scalar loads)
  // the lists cover 256-row tiles; this tile is half qt % 2 of tile qt / 2
  const int qp = qt >> 1, full_bit = 2 * (qt & 1) + 1;
  const int* list = kv_count ? kv_list + (static_cast<size_t>(bm_b) * p.nq + qp) * p.nk : nullptr;
  const int n_entries = kv_count ? kv_count[bm_b * p.nq + qp] : p.nk;
  int n_stages = 2 * n_entries;
  if (n_entries > 0) {
    const int last = list ? (list[n_entries - 1] >> 4) : (p.nk - 1);
    if (last * kTile + kBN >= p.Skv) n_stages -= 1;   // last tile has a single 64-key stage
  }

  // ---- per-thread global->LDS mapping
  // K: kChunks 16-byte chunks, row-major; V: rows 4*vr .. 4*vr+3, columns vCols*vc ..
  // (consecutive lanes take consecutive key groups so the V^T stores spread
  // over all banks)
  const int vr = tid & 15;
  const int vc = tid >> 4;

  unsigned kreg[G::kChunks][4];
  unsigned vreg[4][G::vCols / 2];

  // Stage it covers keys [kv0, kv0 + 64) of list entry it / 2. Entries are
  // (key_tile << 4) | status bits of the two 128-row halves; a tile with no
  // admitted pair in this half is visited as partial (every score masked, so
  // it adds exactly nothing). The entry of stage it + 2 is fetched during
  // stage it (before that stage's K/V prefetch), so its latency is covered by
  // a whole stage and no wait is needed when it is used.
  auto entry_at = [list](int e) -> int { return list ? list[e] : (e << 4); };
  auto stage_kv0 = [](int it, int ent) -> int { return (ent >> 4) * kTile + (it & 1) * kBN; };

  // keys past Skv read as zero (buffer range check)
  auto load_stage = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < G::kChunks; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / (D / 8);
      const int col = (ci % (D / 8)) * 8;
      u32x4 r = buf_load8<F32>(rk, static_cast<unsigned>(kv0 + row) * p.k_sr + col);
#pragma unroll
      for (int j = 0; j < 4; ++j) kreg[i][j] = r[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = kv0 + vr * 4 + i;
      buf_loadN<F32, G::vCols>(rv, static_cast<unsigned>(row) * p.v_sr + vc * G::vCols, vreg[i]);
    }
  };

  auto store_stage = [&](int buf) {
    __bf16* ks = smem + buf * G::stage;
    __bf16* vs = ks + G::kElems;
#pragma unroll
    for (int i = 0; i < G::kChunks; ++i) {
      const int ci = tid + i * kThreads;
      const int row = ci / (D / 8);
      const int col = (ci % (D / 8)) * 8;
      u32x4 r = {kreg[i][0], kreg[i][1], kreg[i][2], kreg[i][3]};
      *reinterpret_cast<u32x4*>(ks + row * G::kStride + col) = r;
    }
    // V^T: keys 4*vr..4*vr+3 of column d go to one 8-byte slot. Within each
    // 16-key chunk the key groups of 4 are placed in the order 0,2,1,3 so that
    // the eight keys one lane half needs for an MFMA are contiguous.
    const int kl = vr * 4;                 // local key (multiple of 4)
    const int a = (kl >> 2) & 3;
    const int pos = (kl & ~15) + 4 * (((a & 1) << 1) | (a >> 1));
#pragma unroll
    for (int c = 0; c < G::vCols; ++c) {
      const int d = vc * G::vCols + c;
      // column c of rows r and r+1: low (even c) or high (odd c) halves, one v_perm each
      const int w = c >> 1;
      const unsigned sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x2 pr = {__builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel),
                  __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel)};
      *reinterpret_cast<u32x2*>(vs + d * G::vStride + pos) = pr;
    }
  };

  // ---- running state: O^T accumulators, row max (log2 units), lane-partial sum
  f32x16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  using SM = ScoreMod<MOD>;
  const int q_pos = q_row + p.va.q_offset;   // position in the key sequence
  if constexpr (MOD == kModRelBias) stage_rel_table(p.va, h, (lds_f32*)(rtab), tid, kThreads);
  const typename SM::Lane sml = [&] {
    typename SM::Lane L = SM::lane(p.va, h, q_pos);
    if constexpr (MOD == kModRelBias) L.tab = (lds_cf32*)(rtab) + p.va.rel_max;
    return L;
  }();
  // document labels of this batch row (document-mask kernels only)
  const int* doc_row = DOCS ? p.va.doc + static_cast<size_t>(b) * p.va.doc_stride : p.va.doc;
  const rsrc_t rdoc = make_rsrc(doc_row, DOCS ? static_cast<unsigned>(p.va.doc_stride) * 4u : 0u);
  const int doc_q = (DOCS && q_ok) ? doc_row[q_pos] : 0;

  int ent_cur = 0, ent_next = 0;   // entries of stages it and it + 1
  if (n_stages > 0) {
    ent_cur = entry_at(0);
    ent_next = n_stages > 1 ? entry_at(1 >> 1) : 0;
    load_stage(stage_kv0(0, ent_cur));
    store_stage(0);
  }
  // Retire every outstanding load here (Q fragments included). Otherwise the
  // wait the compiler places before the first in-loop use of the Q fragments
  // also waits for the next stage's prefetch, which defeats the prefetch.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < n_stages; ++it) {
    const int cur = it & 1;
    const int ent_after = (it + 2 < n_stages) ? entry_at((it + 2) >> 1) : 0;
    const int ent = __builtin_amdgcn_readfirstlane(ent_cur);
    const bool full = ((ent >> full_bit) & 1) != 0;
    const int kv0 = stage_kv0(it, ent);
    const bool more = it + 1 < n_stages;
    if (more) load_stage(stage_kv0(it + 1, __builtin_amdgcn_readfirstlane(ent_next)));
    ent_cur = ent_next;
    ent_next = ent_after;

    const __bf16* ks = smem + cur * G::stage;
    const __bf16* vs = ks + G::kElems;

    // S^T = K Q^T : two 32-key blocks, the two accumulation chains
    // interleaved. The fragment reads are kept 4 ahead of the MFMAs that use
    // them (instruction-group order below), so LDS latency hides behind
    // ~4 x 32 cycles of matrix work instead of stalling each MFMA.
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const __bf16* krow = ks + (kb * 32 + l32) * G::kStride + g * 8;
        bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + c * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x0020, 16, 0);   // the prefetch buffer loads
    __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);    // 4 fragment reads ahead
#pragma unroll
    for (int i = 0; i < 2 * DC - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // 1 fragment read
    }
    __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);    // last 4 MFMAs

    // Scores as 32 scalars (element 16*kb + r holds key kv0 + 32*kb +
    // 8*(r/4) + 4*g + r%4); score_mod in place, then mask_mod in place on
    // partial tiles only.
    float t[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kidx = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        t[kb * 16 + r] = SM::apply(s[kb][r], p.va, sml, kidx - q_pos);
      }
    if (!full) {
      // Branch-free predicate. The four keys 8*i + 4*g + (0..3) of a block are
      // consecutive, so their document labels come in one 16-byte buffer load
      // (keys past Skv read as label 0 but are rejected by the range test).
      const bool causal = p.mask_kind & kMaskCausal;
      const bool window = p.mask_kind & kMaskWindow;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = kv0 + kb * 32 + 8 * i + 4 * g;
          u32x4 lab = {0u, 0u, 0u, 0u};
          if constexpr (DOCS) lab = __builtin_amdgcn_raw_buffer_load_b128(rdoc, static_cast<unsigned>(k0) * 4u, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kidx = k0 + e;
            bool ok = kidx < p.Skv;
            ok &= !causal | (q_pos >= kidx) | (kidx < p.va.prefix);
            ok &= !window | (q_pos - kidx < p.va.window);
            if constexpr (DOCS) ok &= static_cast<int>(lab[e]) == doc_q;
            t[kb * 16 + 4 * i + e] = ok ? t[kb * 16 + 4 * i + e] : -INFINITY;
          }
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, t[i]);
    mx = max_pair32(mx);
    if constexpr (SM::kFoldScale) mx *= p.va.c1;   // raw -> log2 units (c1 > 0)

    // conditional rescale (wave-uniform decision)
    if (__any(q_ok && mx > m_run + kRescaleLog2)) {   // rows past Sq take no part
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float base = (m_run == -INFINITY) ? 0.f : m_run;

    // P = exp2(t - base), rounded to bf16 as the B operand of the second product
    bf16x8 pf[4];
    float ls = 0.f;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const int kb = ch >> 1, r0 = (ch & 1) * 8;
      unsigned w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p0, p1;
        if constexpr (SM::kFoldScale) {
          p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kb * 16 + r0 + 2 * j], p.va.c1, -base));
          p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kb * 16 + r0 + 2 * j + 1], p.va.c1, -base));
        } else {
          p0 = __builtin_amdgcn_exp2f(t[kb * 16 + r0 + 2 * j] - base);
          p1 = __builtin_amdgcn_exp2f(t[kb * 16 + r0 + 2 * j + 1] - base);
        }
        ls += p0 + p1;
        w[j] = pack_bf16(p0, p1);
      }
      u32x4 wv = {w[0], w[1], w[2], w[3]};
      pf[ch] = __builtin_bit_cast(bf16x8, wv);
    }
    l_run += ls;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + l32;
      const __bf16* vrow = vs + d * G::vStride;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + (2 * ch + g) * 8);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], o[db], 0, 0, 0);
      }
    }

    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, LSE, store
  const float l_tot = sum_pair32(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (q_ok) {
    const size_t orow = b * p.o_sb + h * p.o_sh + static_cast<size_t>(q_row) * p.o_sr;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        const float x0 = o[db][4 * i] * inv, x1 = o[db][4 * i + 1] * inv;
        const float x2 = o[db][4 * i + 2] * inv, x3 = o[db][4 * i + 3] * inv;
        if constexpr (F32) {
          f32x4 vv = {x0, x1, x2, x3};
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + orow + d0) = vv;
        } else {
          u32x2 vv = {pack_bf16(x0, x1), pack_bf16(x2, x3)};
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(p.out) + orow + d0) = vv;
        }
      }
    }
    if (p.lse && g == 0) {
      p.lse[q_head + q_row] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int MOD, bool F32, bool DOCS>
hipError_t launch_t(const FwdLaunch& p, hipStream_t stream) {
  const int nq = (p.Sq + kBM - 1) / kBM;
  const long long total = static_cast<long long>(p.B) * p.H * nq;
  const long long per = (total + kXcds - 1) / kXcds;
  dim3 grid(static_cast<unsigned>(per * kXcds));
  note_launch("attn_fwd_kernel<%d, %d, %s, %s> grid %lld x %d", D, MOD, F32 ? "true" : "false",
              DOCS ? "true" : "false", per * kXcds, kThreads);
  hipLaunchKernelGGL((attn_fwd_kernel<D, MOD, F32, DOCS>), grid, dim3(kThreads), 0, stream, p,
                     p.kv_count, p.kv_list);
  return hipGetLastError();
}

template <int D, bool F32, bool DOCS>
hipError_t launch_mod(const FwdLaunch& p, hipStream_t stream) {
  switch (p.mod_kind) {
    case kModNone: return launch_t<D, kModNone, F32, DOCS>(p, stream);
    case kModAlibi: return launch_t<D, kModAlibi, F32, DOCS>(p, stream);
    case kModSoftcap: return launch_t<D, kModSoftcap, F32, DOCS>(p, stream);
    case kModRelBias: return launch_t<D, kModRelBias, F32, DOCS>(p, stream);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const FwdLaunch& p, hipStream_t stream) {
  const bool docs = p.mask_kind & kMaskDocument;
  if (p.is_fp32) return docs ? launch_mod<D, true, true>(p, stream) : launch_mod<D, true, false>(p, stream);
  return docs ? launch_mod<D, false, true>(p, stream) : launch_mod<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdLaunch& p, hipStream_t stream) {
  if (!p.is_fp32 && p.nk <= kPairMaxKeyTiles) return launch_attn_fwd_pp(p, stream);
  if (p.D == 128) return launch_d<128>(p, stream);
  if (p.D == 64) return launch_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
