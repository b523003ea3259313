// block_mask.hip - block-mask builder: classify every (query half-tile, key
// tile) pair of a mask_mod as empty, partial or full, and write for each
// 256-row query tile the ascending list of key tiles that are non-empty for
// at least one of its two 128-row halves, with the class of each half.
//
// FlexAttention's user-supplied score and mask functions (PyTorch
// FlexAttention FA4-backend post; NextVector FlexAttention article, body) let
// masked structure be known ahead of the kernel. Skipping empty tiles and dropping the per-element test on
// full ones is how a sparse variant (sliding window, document packing) runs at
// dense-tile speed on the tiles it does compute.
//
// Query rows stand at positions row + q_offset. The causal and window parts
// act on the difference d = q - k of positions, and over a rectangle of
// positions d takes every integer between its extremes, so those two parts are
// classified exactly from the rectangle's corners. Under a prefix-LM mask the
// keys below the prefix drop the causal part: a tile is split at the prefix
// and each side classified exactly, the tile being full when both sides are
// and empty when both are. The document part is classified from the label
// ranges of the query rows and of the keys where those decide it (disjoint
// ranges: empty; one shared label: the positional class); the pairs they
// leave open are decided exactly by a test over the key tile's label runs.
// So every class equals the one a pair-by-pair test would give. Keys at or
// past Skv never count as admitted, so a tile that reaches past Skv is at
// most partial.
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

// Exact "empty or partial" test of one (128-row half, key tile) pair under a
// document mask, by the whole wave. Every mask part but the documents admits,
// for a query at position q, one interval of key positions: from
// q - window + 1 (window) or 0, up to max(q, prefix - 1) (causal, with the
// prefix-LM relaxation: k <= q or k < prefix) or Skv - 1. The lane's rows
// carry their labels lab_r[] and intervals [lo_r[], hi_r[]] (an empty
// interval for a row past Sq). The tile's keys fall into runs of equal
// label; a pair is admitted iff some row's label equals a run's label and its
// interval meets that run. Lanes hold keys ka + lane and ka + 64 + lane, run
// starts are found with a ballot, and the runs are walked in order on the
// scalar unit, so the cost is a few instructions per run, not per pair.
// The labels come from tile_labels, issued for several tiles before the
// first walk so that their loads are in flight together.
struct TileLabels {
  int l0, l1;   // labels of keys ka + lane and ka + 64 + lane (0 past the tile)
};
__device__ inline TileLabels tile_labels(const int* doc, int ka, int kb, int lane) {
  const int n = kb - ka + 1;
  return {lane < n ? doc[ka + lane] : 0, lane + 64 < n ? doc[ka + 64 + lane] : 0};
}
__device__ bool half_tile_has_pair(const TileLabels& t, int ka, int kb, int lane, const int (&lab_r)[2],
                                   const int (&lo_r)[2], const int (&hi_r)[2]) {
  const int n = kb - ka + 1;   // keys in the tile (1..128)
  const bool in0 = lane < n, in1 = lane + 64 < n;
  const int l0 = t.l0, l1 = t.l1;
  // label of the key before each of the lane's two keys
  const int prev0 = __shfl(l0, lane == 0 ? 0 : lane - 1);
  const int prev1 = lane == 0 ? __shfl(l0, 63) : __shfl(l1, lane - 1);
  uint64_t s0 = __ballot(in0 && (lane == 0 || l0 != prev0));
  uint64_t s1 = __ballot(in1 && l1 != prev1);
  bool hit = false;
  while (s0 | s1) {
    int st;
    if (s0) {
      st = __builtin_ctzll(s0);
      s0 &= s0 - 1;
    } else {
      st = 64 + __builtin_ctzll(s1);
      s1 &= s1 - 1;
    }
    const int nx = s0 ? __builtin_ctzll(s0) : s1 ? 64 + __builtin_ctzll(s1) : n;
    const int label = st < 64 ? __builtin_amdgcn_readlane(l0, st) : __builtin_amdgcn_readlane(l1, st - 64);
    const int rs = ka + st, re = ka + nx - 1;   // the run's key positions
#pragma unroll
    for (int i = 0; i < 2; ++i)
      hit = hit || (lab_r[i] == label && max(lo_r[i], rs) <= min(hi_r[i], re));
  }
  return __ballot(hit) != 0;
}

// One wave per (batch row, 256-row query tile); each lane classifies one key
// tile (64 per pass) for both 128-row halves, and the non-empty tiles are
// compacted in order with a ballot.
//
// Per half, causal and window give the class cls_d exactly from the corners.
// Documents: with the label ranges of the half's rows [dq_min, dq_max] and of
// the tile's keys [dk_min, dk_max], disjoint ranges mean empty and one shared
// label means cls_d. A full tile needs every pair to share its label, which
// the ranges decide exactly. Ranges that overlap without one shared label
// leave "empty or partial" open (never "full": some pair then has two
// labels); half_tile_has_pair decides those pairs.
// (Few workgroups run at once, so the kernel may take the registers that keep
// all of a tile's label loads in flight.)
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void block_mask_kernel(MaskLaunch p) {
  const int qp = blockIdx.x;
  const int bb = blockIdx.y;
  const int lane = threadIdx.x;
  const bool causal = p.mask_kind & kMaskCausal;
  const bool window = p.mask_kind & kMaskWindow;
  const bool docs = p.mask_kind & kMaskDocument;
  const int* doc = docs ? p.doc + static_cast<size_t>(bb) * p.doc_stride : nullptr;

  // positions of each half's rows
  int q_lo[2], q_hi[2], dq_min[2] = {0, 0}, dq_max[2] = {0, 0};
  bool live[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r_lo = qp * 2 * kTile + hf * kTile;
    live[hf] = r_lo < p.Sq;
    q_lo[hf] = r_lo + p.q_offset;
    q_hi[hf] = min(p.Sq, r_lo + kTile) - 1 + p.q_offset;
    if (docs && live[hf]) label_range(doc, q_lo[hf], q_hi[hf], lane, dq_min[hf], dq_max[hf]);
  }

  // admitted differences d = q - k form the interval [lo_d, hi_d]; keys
  // below the prefix take [lo_p, hi_d] (no causal bound)
  const long long lo_d = causal ? 0 : -(1LL << 40);
  const long long lo_p = -(1LL << 40);
  const long long hi_d = window ? static_cast<long long>(p.window) - 1 : (1LL << 40);
  const int prefix = causal ? p.prefix : 0;

  // for the exact document test: rows r_lo + lane and r_lo + 64 + lane of
  // each half, with their labels and admitted key intervals
  int lab_r[2][2] = {{0, 0}, {0, 0}}, lo_r[2][2], hi_r[2][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = qp * 2 * kTile + hf * kTile + 64 * i + lane;
      lo_r[hf][i] = 1;   // empty interval unless the row exists
      hi_r[hf][i] = 0;
      if (docs && row < p.Sq) {
        const int q = row + p.q_offset;
        lab_r[hf][i] = doc[q];
        const long long lo = window ? static_cast<long long>(q) - p.window + 1 : 0;
        const long long hi = causal ? max(q, prefix - 1) : p.Skv - 1;
        lo_r[hf][i] = static_cast<int>(max(lo, 0LL));
        hi_r[hf][i] = static_cast<int>(min(hi, static_cast<long long>(p.Skv) - 1));
      }
    }
  // class of rows [qa, qb] x keys [ka, kb] under d in [lo, hi]
  auto rect = [&](int qa, int qb, int ka, int kb, long long lo) -> int {
    const long long dmin = static_cast<long long>(qa) - kb;
    const long long dmax = static_cast<long long>(qb) - ka;
    if (dmax < lo || dmin > hi_d) return kEmpty;
    if (dmin >= lo && dmax <= hi_d) return kFull;
    return kPartial;
  };

  int* out = p.kv_list + (static_cast<size_t>(bb) * p.nq + qp) * p.nk;
  int n = 0;
  for (int kt0 = 0; kt0 < p.nk; kt0 += 64) {
    const int kt = kt0 + lane;
    const bool valid = kt < p.nk;
    const int k_lo = valid ? kt * kTile : 0;
    const int k_hi = valid ? min(p.Skv, k_lo + kTile) - 1 : 0;
    const bool in_range = k_lo + kTile <= p.Skv;

    int cls[2];
    bool need_labels = false;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (!valid || !live[hf]) {
        cls[hf] = kEmpty;
      } else if (k_lo >= prefix) {
        cls[hf] = rect(q_lo[hf], q_hi[hf], k_lo, k_hi, lo_d);
      } else if (k_hi < prefix) {
        cls[hf] = rect(q_lo[hf], q_hi[hf], k_lo, k_hi, lo_p);
      } else {
        const int a = rect(q_lo[hf], q_hi[hf], k_lo, prefix - 1, lo_p);
        const int c = rect(q_lo[hf], q_hi[hf], prefix, k_hi, lo_d);
        cls[hf] = (a == kEmpty && c == kEmpty) ? kEmpty
                  : (a == kFull && c == kFull) ? kFull : kPartial;
      }
      need_labels = need_labels || cls[hf] != kEmpty;
    }
    if (docs && need_labels) {
      int dk_min = 0x7fffffff, dk_max = -0x7fffffff - 1;
      int k = k_lo;
      if (in_range && (reinterpret_cast<uintptr_t>(doc + k_lo) & 15) == 0) {
        // a whole tile: 32 aligned 16-byte loads, all in flight
        const int4* v4 = reinterpret_cast<const int4*>(doc + k_lo);
#pragma unroll
        for (int i = 0; i < kTile / 4; ++i) {
          const int4 v = v4[i];
          dk_min = min(dk_min, min(min(v.x, v.y), min(v.z, v.w)));
          dk_max = max(dk_max, max(max(v.x, v.y), max(v.z, v.w)));
        }
        k = k_hi + 1;
      }
      for (; k <= k_hi; ++k) {
        const int v = doc[k];
        dk_min = min(dk_min, v);
        dk_max = max(dk_max, v);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (cls[hf] == kEmpty) continue;
        if (dq_max[hf] < dk_min || dk_max < dq_min[hf]) cls[hf] = kEmpty;
        else if (!(dq_min[hf] == dq_max[hf] && dk_min == dk_max && dq_min[hf] == dk_min)) cls[hf] = kUnknown;
      }
    }

    // Pairs the label ranges leave open: decided by the whole wave, the open
    // (tile, half) pairs of this pass in order, kBatch at a time (the labels
    // of a batch's tiles are loaded together, then each tile is walked).
    if (docs) {
      constexpr int kBatch = 8;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint64_t open = __ballot(cls[hf] == kUnknown);
        uint64_t found = 0;
        while (open) {
          int js[kBatch];
          TileLabels tl[kBatch];
#pragma unroll
          for (int q = 0; q < kBatch; ++q) {
            js[q] = -1;
            if (open) {
              js[q] = __builtin_ctzll(open);
              open &= open - 1;
              const int ka = (kt0 + js[q]) * kTile;
              tl[q] = tile_labels(doc, ka, min(p.Skv, ka + kTile) - 1, lane);
            }
          }
#pragma unroll
          for (int q = 0; q < kBatch; ++q) {
            if (js[q] < 0) break;
            const int ka = (kt0 + js[q]) * kTile;
            if (half_tile_has_pair(tl[q], ka, min(p.Skv, ka + kTile) - 1, lane, lab_r[hf], lo_r[hf], hi_r[hf]))
              found |= 1ull << js[q];
          }
        }
        if (cls[hf] == kUnknown) cls[hf] = ((found >> lane) & 1) ? kPartial : kEmpty;
      }
    }

    int bits = 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      int c = cls[hf];
      if (c == kFull && !in_range) c = kPartial;
      if (c != kEmpty) bits |= (c == kFull ? 3 : 1) << (2 * hf);
    }
    const uint64_t have = __ballot(bits != 0);
    const int before = __builtin_popcountll(have & ((1ull << lane) - 1ull));
    if (bits) out[n + before] = (kt << 4) | bits;
    n += __builtin_popcountll(have);
  }
  if (lane == 0) p.kv_count[bb * p.nq + qp] = n;
}

}  // namespace

hipError_t launch_block_mask(const MaskLaunch& p, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(p.nq), static_cast<unsigned>(p.num_b));
  note_launch("block_mask_kernel grid %d x %d x 64", p.nq, p.num_b);
  hipLaunchKernelGGL(block_mask_kernel, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
