// Measured matrix-core peaks of the GPU this runs on.
//
// Each kernel does nothing but back-to-back MFMAs on register operands, with
// several independent accumulator chains per wave so the matrix core never
// waits on a result, and 8 waves per SIMD so issue never starves it.  The
// achieved rate is the practical ceiling a hand-written kernel of the same
// instruction can reach, the second denominator (beside the datasheet peak)
// for a roofline fraction.  Measurement support only: the attention library
// does not link or call this.
//
// C ABI (libslapeak.so):
//   int slapeak_mfma(int kind, int iters, int grid, int *out, hipStream_t st)
//     kind 0: v_mfma_i32_16x16x64_i8    1: v_mfma_i32_32x32x32_i8
//          2: v_mfma_f32_16x16x32_bf16  3: v_mfma_f32_32x32x16_bf16
//     grid workgroups of 256 threads (4 waves), each wave iters rounds of
//     SLAPEAK_CHAINS(kind) MFMAs; out: device int32[grid * 4], one word per
//     wave (a digest of its accumulators, so no chain is dead code).
//     Returns 0, 1 for a bad argument, 2 for a launch error.
//   long long slapeak_mfma_ops(int kind, int iters, int grid)
//     integer ops / flops one such launch executes (2 M N K per MFMA).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slapeak {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// shape of each kind: M N K, accumulator chains per wave
constexpr int kM[4] = {16, 32, 16, 32};
constexpr int kN[4] = {16, 32, 16, 32};
constexpr int kK[4] = {64, 32, 32, 16};
constexpr int kChains[4] = {8, 4, 8, 4};

template <int KIND> struct Acc;
template <> struct Acc<0> { typedef v4i T; };
template <> struct Acc<1> { typedef v16i T; };
template <> struct Acc<2> { typedef v4f T; };
template <> struct Acc<3> { typedef v16f T; };

template <int KIND>
__device__ __forceinline__ typename Acc<KIND>::T mma(v4i a, v4i b, typename Acc<KIND>::T c) {
  if constexpr (KIND == 0) return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  if constexpr (KIND == 1) return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  if constexpr (KIND == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  if constexpr (KIND == 3)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <int KIND>
__global__ __launch_bounds__(256) void k_peak(int iters, int *__restrict__ out) {
  constexpr int C = kChains[KIND];
  typedef typename Acc<KIND>::T A;
  const int tid = threadIdx.x;
  // small operands (bf16 about 2^-6, int8 bytes 0..3): finite sums for any iters
  const uint32_t u = 0x3C803C80u + (uint32_t)(tid & 3);
  const uint32_t ib = 0x01010101u * (uint32_t)(tid & 3);
  const v4i a = (KIND < 2) ? v4i{(int)ib, (int)(ib ^ 1u), (int)ib, (int)(ib ^ 2u)}
                           : v4i{(int)u, (int)u, (int)(u ^ 1u), (int)u};
  const v4i b = a.yzwx;
  // eight (16x16 kinds) or four (32x32 kinds) chains in named registers,
  // started from different values so the compiler cannot merge them
  A c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
  c1[0] = 1, c2[0] = 2, c3[0] = 3, c4[0] = 4, c5[0] = 5, c6[0] = 6, c7[0] = 7;
  for (int it = 0; it < iters; ++it) {
    c0 = mma<KIND>(a, b, c0);
    c1 = mma<KIND>(a, b, c1);
    c2 = mma<KIND>(a, b, c2);
    c3 = mma<KIND>(a, b, c3);
    if constexpr (C == 8) {
      c4 = mma<KIND>(a, b, c4);
      c5 = mma<KIND>(a, b, c5);
      c6 = mma<KIND>(a, b, c6);
      c7 = mma<KIND>(a, b, c7);
    }
  }
  // every element of every chain feeds the digest (else the compiler keeps
  // only the elements read and overlaps the chains' registers)
  constexpr int E = sizeof(A) / 4;
  int dig = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int x = __builtin_bit_cast(int, c0[e]) ^ __builtin_bit_cast(int, c1[e]) ^
            __builtin_bit_cast(int, c2[e]) ^ __builtin_bit_cast(int, c3[e]);
    if constexpr (C == 8)
      x ^= __builtin_bit_cast(int, c4[e]) ^ __builtin_bit_cast(int, c5[e]) ^
           __builtin_bit_cast(int, c6[e]) ^ __builtin_bit_cast(int, c7[e]);
    dig = dig * 3 + x;
  }
  if ((tid & 63) == 0) out[blockIdx.x * 4 + (tid >> 6)] = dig;
}

}  // namespace slapeak

extern "C" long long slapeak_mfma_ops(int kind, int iters, int grid) {
  if (kind < 0 || kind > 3 || iters < 0 || grid < 0) return -1;
  using namespace slapeak;
  return 2LL * kM[kind] * kN[kind] * kK[kind] * kChains[kind] * iters * 4LL * grid;
}

extern "C" int slapeak_mfma(int kind, int iters, int grid, int *out, hipStream_t st) {
  using namespace slapeak;
  if (kind < 0 || kind > 3 || iters < 1 || grid < 1 || !out) return 1;
  switch (kind) {
    case 0: k_peak<0><<<grid, 256, 0, st>>>(iters, out); break;
    case 1: k_peak<1><<<grid, 256, 0, st>>>(iters, out); break;
    case 2: k_peak<2><<<grid, 256, 0, st>>>(iters, out); break;
    default: k_peak<3><<<grid, 256, 0, st>>>(iters, out); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
