// block_mask.hip - block-mask builder: classify every (query half-tile, key
// tile) pair of a mask_mod as empty, partial or full, and write for each
// 256-row query tile the ascending list of key tiles that are non-empty for
// at least one of its two 128-row halves, with the class of each half.
//
// FlexAttention's score/mask modifications (PyTorch FlexAttention FA4-backend
// post; NextVector FlexAttention article, body) let masked structure be known
// ahead of the kernel. Skipping empty tiles and dropping the per-element test on
// full ones is how a sparse variant (sliding window, document packing) runs at
// dense-tile speed on the tiles it does compute.
//
// One wave per (batch row, 256-row query tile). The causal and window parts act on the
// difference d = q - k, and over a rectangle of positions d takes every integer
// between its extremes, so those two parts are classified exactly from the
// rectangle's corners. The document part is classified from the label range of
// the query rows and of the keys; when that is inconclusive the wave tests every
// pair of the tile. Keys at or past Skv never count as admitted, so a tile that
// reaches past Skv is at most partial.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "variants.h"

namespace fa {
namespace {

constexpr int kTile = 128;

enum : int { kEmpty = 0, kPartial = 1, kFull = 2, kUnknown = 3 };

__device__ inline int wave_min(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ inline int wave_max(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Label range of positions [lo, hi] (inclusive, non-empty) of one batch row.
__device__ inline void label_range(const int* doc, int lo, int hi, int lane, int& mn, int& mx) {
  int a = 0x7fffffff, b = -0x7fffffff - 1;
  for (int i = lo + lane; i <= hi; i += 64) {
    const int v = doc[i];
    a = min(a, v);
    b = max(b, v);
  }
  mn = wave_min(a);
  mx = wave_max(b);
}

// Class of the rectangle (query rows [q_lo, q_hi]) x (keys [k_lo, k_hi]),
// both non-empty. cls_d is the class under causal/window alone; dq_* and
// dk_* are the label ranges of the rows and of the keys (documents only).
__device__ inline int classify(const MaskLaunch& p, const int* doc, int lane, int q_lo, int q_hi,
                               int k_lo, int k_hi, int cls_d, int dq_min, int dq_max, int dk_min,
                               int dk_max) {
  int cls = cls_d;
  if (cls != kEmpty && doc) {
    if (dq_max < dk_min || dk_max < dq_min) cls = kEmpty;
    else if (dq_min == dq_max && dk_min == dk_max && dq_min == dk_min) cls = cls_d;  // one shared document
    else cls = kUnknown;
  }
  if (cls == kUnknown) {
    // test every in-range pair: lane takes query rows q_lo+lane and q_lo+64+lane
    bool any = false, all = true;
    for (int r = 0; r < 2; ++r) {
      const int q = q_lo + r * 64 + lane;
      if (q > q_hi) continue;
      const int dq = doc[q];
      for (int k = k_lo; k <= k_hi; ++k) {
        const bool ok = admit(p.mask_kind, q, k, p.window, doc, dq);
        any = any || ok;
        all = all && ok;
      }
    }
    const bool w_any = __any(any);
    const bool w_all = __all(all);
    cls = !w_any ? kEmpty : (w_all ? kFull : kPartial);
  }
  return cls;
}

// One wave per (batch row, 256-row query tile); the two 128-row halves are
// classified separately and share one list.
__global__ __launch_bounds__(64) void block_mask_kernel(MaskLaunch p) {
  const int qp = blockIdx.x;
  const int bb = blockIdx.y;
  const int lane = threadIdx.x;
  const bool causal = p.mask_kind & kMaskCausal;
  const bool window = p.mask_kind & kMaskWindow;
  const bool docs = p.mask_kind & kMaskDocument;
  const int* doc = docs ? p.doc + static_cast<size_t>(bb) * p.doc_stride : nullptr;

  int q_lo[2], q_hi[2], dq_min[2] = {0, 0}, dq_max[2] = {0, 0};
  bool live[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    q_lo[hf] = qp * 2 * kTile + hf * kTile;
    q_hi[hf] = min(p.Sq, q_lo[hf] + kTile) - 1;
    live[hf] = q_lo[hf] < p.Sq;
    if (docs && live[hf]) label_range(doc, q_lo[hf], q_hi[hf], lane, dq_min[hf], dq_max[hf]);
  }

  // admitted differences d = q - k form the interval [lo_d, hi_d]
  const long long lo_d = causal ? 0 : -(1LL << 40);
  const long long hi_d = window ? static_cast<long long>(p.window) - 1 : (1LL << 40);

  int* out = p.kv_list + (static_cast<size_t>(bb) * p.nq + qp) * p.nk;
  int n = 0;
  for (int kt = 0; kt < p.nk; ++kt) {
    const int k_lo = kt * kTile;
    const int k_hi = min(p.Skv, k_lo + kTile) - 1;
    const bool in_range = k_lo + kTile <= p.Skv;

    // causal and window: over a half, d ranges over [q_lo - k_hi, q_hi - k_lo]
    int cls_d[2];
    bool need_labels = false;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const long long dmin = static_cast<long long>(q_lo[hf]) - k_hi;
      const long long dmax = static_cast<long long>(q_hi[hf]) - k_lo;
      if (!live[hf] || dmax < lo_d || dmin > hi_d) cls_d[hf] = kEmpty;
      else if (dmin >= lo_d && dmax <= hi_d) cls_d[hf] = kFull;
      else cls_d[hf] = kPartial;
      need_labels = need_labels || cls_d[hf] != kEmpty;
    }
    int dk_min = 0, dk_max = 0;
    if (docs && need_labels) label_range(doc, k_lo, k_hi, lane, dk_min, dk_max);

    int bits = 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      int cls = classify(p, doc, lane, q_lo[hf], q_hi[hf], k_lo, k_hi, cls_d[hf], dq_min[hf],
                         dq_max[hf], dk_min, dk_max);
      if (cls == kFull && !in_range) cls = kPartial;
      if (cls != kEmpty) bits |= (cls == kFull ? 3 : 1) << (2 * hf);
    }
    if (bits) {
      if (lane == 0) out[n] = (kt << 4) | bits;
      ++n;
    }
  }
  if (lane == 0) p.kv_count[bb * p.nq + qp] = n;
}

}  // namespace

hipError_t launch_block_mask(const MaskLaunch& p, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(p.nq), static_cast<unsigned>(p.num_b));
  hipLaunchKernelGGL(block_mask_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
