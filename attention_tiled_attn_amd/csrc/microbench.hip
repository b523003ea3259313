// microbench.hip - microbenchmarks of the gfx950 units the attention kernels
// lean on: the bf16 matrix cores, the exponential, plain vector issue, the
// interference between the two waves of a SIMD, LDS fragment reads, and HBM.
// They fix the figures the kernels are judged by beside the published peaks:
// what the matrix cores sustain at the clock the chip actually runs, how many
// exponentials a CU retires per clock, and what one vector instruction of the
// other wave costs a wave that is multiplying.
//
// A units kernel runs a fixed loop in every wave and records per wave the
// shader-clock cycles (s_memtime) and the 100 MHz real-time counter
// (s_memrealtime) around it, so rates come out per clock and per second, and
// the clock itself as their ratio. Each workgroup asks for more than half of
// a CU's LDS, so every workgroup has a CU to itself; waves w and w + 4 of a
// workgroup share SIMD w % 4.
//
// C ABI (libflexattn_mb.so; test infrastructure for measurement, not part of
// the attention library):
//   int flexattn_mb_units(int kind, int waves_per_simd, int iters,
//                         int iters_vec, int workgroups,
//                         unsigned long long* rec, float* sink, void* stream)
//     kind: 0 MFMA (v_mfma_f32_32x32x16_bf16, 8 independent chains per wave)
//           1 EXP  (v_exp_f32, 16 independent chains per wave)
//           2 FMA  (v_fma_f32, 16 independent chains per wave)
//           3 MFMA in waves 0-3 beside FMA in waves 4-7 (waves_per_simd 2)
//           4 MFMA in waves 0-3 beside EXP in waves 4-7 (waves_per_simd 2)
//     iters: loop steps of each wave; in kinds 3 and 4 the vector waves run
//           iters_vec steps (chosen so that they outlast the MFMA waves)
//           5 LDS  (ds_read_b128, 8 reads of distinct 1 KB rows per step)
//           6 LDS  (ds_read_b64_tr_b16, 16 transposing reads per step)
//           7 EXP and FMA in one wave (16 + 32 per step, independent)
//     rec : device, 3 x u64 per wave (cycles, real-time ticks, operations)
//           for workgroups x 4 x waves_per_simd waves
//     sink: device, one float per workgroup (keeps the loops' results alive)
//   int flexattn_mb_read(const void* src, unsigned long long bytes,
//                        float* sink, int workgroups, void* stream)
//     reads `bytes` (a multiple of 16) once with 16-byte loads; sink holds
//     4 floats per workgroup (one per wave)
//   int flexattn_mb_copy(const void* src, void* dst, unsigned long long bytes,
//                        int workgroups, void* stream)
// Return 0, or -1 for a bad argument, -2 for a launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsPad = 96 * 1024;   // dynamic LDS per workgroup: one per CU

__device__ inline void mfma_loop(int iters, float& out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * (lane + i));
    b[i] = static_cast<__bf16>(0.002f * (lane - i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out = s;
}

__device__ inline void exp_loop(int iters, float& out) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0.01f * (j + (threadIdx.x & 63));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);   // stays in (0, 1]
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  out = s;
}

__device__ inline void fma_loop(int iters, float m, float c, float& out) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0.01f * (j + (threadIdx.x & 63));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  out = s;
}

__device__ inline void lds_loop(int iters, const unsigned char* lds, float& out) {
  typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
  const int lane = threadIdx.x & 63;
  // 8 rows of 1 KB per step, 8 KB apart; lane i reads bytes 16 i .. 16 i + 15
  // of a row (64 lanes x 16 bytes: free of bank conflicts). The rows move by
  // 1 KB between steps, and a compiler memory barrier per step keeps every
  // read inside the loop.
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");
    const unsigned base = (static_cast<unsigned>(lane) << 4) | ((static_cast<unsigned>(it) & 1u) << 10);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const u32x4 v1 = *(lds_u32x4*)(lds + base + j * 8192);
      const u32x4 v2 = *(lds_u32x4*)(lds + base + (j + 1) * 8192);
      acc += v1 + v2;
    }
  }
  out = static_cast<float>(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// The same through ds_read_b64_tr_b16 (the transposing read of the V
// fragments): 16 reads of 512 bytes per step. Lane l reads 8 bytes of row
// 4 (l / 16) + (l % 16) / 4 at byte 8 (l % 4); rows are 288 bytes apart, so
// the four rows a 16-lane group reads start 32 bytes apart in the banks and
// do not conflict (the attention kernels get the same from their chunk
// permutation of 256-byte rows).
__device__ inline void lds_tr_loop(int iters, const unsigned char* lds, float& out) {
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const int lane = threadIdx.x & 63;
  const unsigned lo = static_cast<unsigned>(((lane >> 4) * 4 + ((lane & 15) >> 2)) * 288 + (lane & 3) * 8);
  i16x4_t acc = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");
    const unsigned base = lo | ((static_cast<unsigned>(it) & 1u) << 12);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc += __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds + base + (j & 7) * 8192 + (j >> 3) * 32));
  }
  out = static_cast<float>(acc[0] + acc[1] + acc[2] + acc[3]);
}

// One wave mixing both: 16 exponentials and 32 FMAs per step, independent
// of each other (does a wave issue vector work while its exponentials run?).
__device__ inline void exp_fma_loop(int iters, float m, float c, float& out) {
  float x[16], y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = y[j] = 0.01f * (j + (threadIdx.x & 63));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[j] = __builtin_amdgcn_exp2f(-x[j]);
      y[j] = __builtin_fmaf(__builtin_fmaf(y[j], m, c), m, c);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j] + y[j];
  out = s;
}

__global__ __launch_bounds__(512) void mb_units_kernel(int kind, int iters, int iters_vec, float m, float c,
                                                        unsigned long long* rec, float* sink) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  float r = 0.f;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long ops = 0;
  const bool mfma_wave = kind == 0 || ((kind == 3 || kind == 4) && wave < 4);
  if (mfma_wave) {
    mfma_loop(iters, r);
    ops = 8ull * iters;
  } else if (kind == 1 || kind == 4) {
    const int n = kind == 4 ? iters_vec : iters;
    exp_loop(n, r);
    ops = 16ull * n;
  } else if (kind == 2 || kind == 3) {
    const int n = kind == 3 ? iters_vec : iters;
    fma_loop(n, m, c, r);
    ops = 16ull * n;
  } else if (kind == 5) {
    lds_loop(iters, lds, r);
    ops = 8ull * iters;
  } else if (kind == 6) {
    lds_tr_loop(iters, lds, r);
    ops = 16ull * iters;
  } else if (kind == 7) {
    exp_fma_loop(iters, m, c, r);
    ops = 48ull * iters;
  }
  // every operation has retired before the second reading
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" : "+v"(r));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long w1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    unsigned long long* o = rec + 3ull * (static_cast<unsigned long long>(blockIdx.x) * waves + wave);
    o[0] = t1 - t0;
    o[1] = w1 - w0;
    o[2] = ops;
  }
  // keep the loops' results (a per-workgroup sum, written by one lane)
  __shared__ float part[8];
  float s = r;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < waves; ++i) t += part[i];
    sink[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void mb_read_kernel(const f32x4* __restrict__ src, unsigned long long n,
                                                       float* sink) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const unsigned long long stride = static_cast<unsigned long long>(gridDim.x) * blockDim.x;
  for (unsigned long long i = static_cast<unsigned long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    acc += src[i];
  float s = acc[0] + acc[1] + acc[2] + acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(256) void mb_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                       unsigned long long n) {
  const unsigned long long stride = static_cast<unsigned long long>(gridDim.x) * blockDim.x;
  for (unsigned long long i = static_cast<unsigned long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

int flexattn_mb_units(int kind, int waves_per_simd, int iters, int iters_vec, int workgroups,
                      unsigned long long* rec, float* sink, void* stream) {
  if (kind < 0 || kind > 7 || waves_per_simd < 1 || waves_per_simd > 2 || iters < 1 || iters_vec < 1 ||
      workgroups < 1 || workgroups > 65536 || !rec || !sink)
    return -1;
  if ((kind == 3 || kind == 4) && waves_per_simd != 2) return -1;
  static bool lds_set = false;
  if (!lds_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(mb_units_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsPad) != hipSuccess)
      return -2;
    lds_set = true;
  }
  // c = 0.5 (1 - m) keeps x = m x + c inside [0, 1]
  const float m = 0.999f, c = 0.0005f;
  hipLaunchKernelGGL(mb_units_kernel, dim3(workgroups), dim3(256 * waves_per_simd), kLdsPad,
                     static_cast<hipStream_t>(stream), kind, iters, iters_vec, m, c, rec, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int flexattn_mb_read(const void* src, unsigned long long bytes, float* sink, int workgroups, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || workgroups < 1 || workgroups > 65536) return -1;
  hipLaunchKernelGGL(mb_read_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int flexattn_mb_copy(const void* src, void* dst, unsigned long long bytes, int workgroups, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 || workgroups < 1 || workgroups > 65536) return -1;
  hipLaunchKernelGGL(mb_copy_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
