// variant_args.h - the variants' constants and per-call arguments, shared by
// the host side of the library (api.cpp) and the kernels. Plain C++: no
// device code, so that the C ABI also builds with a host compiler (the
// sanitizer build of the argument checks).
#pragma once

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum : int { kMaskCausal = 1, kMaskWindow = 2, kMaskDocument = 4, kMaskPrefix = 8 };
enum : int { kModNone = 0, kModAlibi = 1, kModSoftcap = 2, kModRelBias = 3 };
constexpr int kRelMax = 1023;                 // largest clip distance of a bias table
constexpr int kRelCap = 2 * kRelMax + 2;      // table entries kept in LDS

// Per-call constants the functors read. Filled on the host.
struct VariantArgs {
  float c1;          // scale * log2(e)
  float sc_in;       // softcap: 2 * log2(e) * scale / cap
  float sc_out;      // softcap: cap * log2(e)
  int window;        // sliding window (keys with q - k < window are kept)
  const float* slopes;  // ALiBi slopes [H]
  const int* doc;       // document labels [B][doc_stride]
  int doc_stride;
  int q_offset;      // position of query row 0 in the key sequence
  int prefix;        // causal part admits keys below it too (0 = plain causal)
  const float* rel_bias;   // relative-bias tables [H][2 rel_max + 1]
  int rel_max;             // clip distance R
};

}  // namespace fa
