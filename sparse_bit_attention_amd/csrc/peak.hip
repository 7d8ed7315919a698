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
//   int slapeak_issue(int kind, int wps, int iters, int grid, long long *cyc,
//                     int *dig, hipStream_t st)
//     Issue-rate probe: grid workgroups of 8 waves, of which the first
//     4 * wps (wps = 1 or 2 waves per SIMD) run iters rounds of one
//     instruction mix, the rest exit at once.  kind 0: 8 independent
//     v_fma_f32; 1: 8 independent v_exp_f32; 2: 8 v_mfma_f32_16x16x32_bf16
//     (8 chains); 3: the same 8 MFMAs, each followed by two independent
//     v_fma_f32.  cyc: device int64[grid * 8 * 4], per wave the shader
//     clock (s_memtime) and the 100 MHz real-time clock (s_memrealtime) at
//     the start and at the end of its rounds (all 0 for waves that exited);
//     dig: device int32[grid * 8] digests.  Returns 0, 1 for a bad argument,
//     2 for a launch error.
//   int slapeak_stream(int kind, int waves, int iters, int grid, const void *buf,
//                      long long *cyc, int *dig, hipStream_t st)
//     Operand-delivery probe: grid workgroups of 8 waves, of which the first
//     `waves` (1..8) run iters rounds; in round it each reads 8 KiB (16 bytes
//     per lane, 8 pieces) alternating between two 8 KiB halves of its
//     workgroup's 16 KiB.  kind 0: global loads from buf (device, at least
//     grid * 16 KiB, L1-resident after the first rounds); kind 1: LDS reads
//     (buf unused, may be null).  cyc: device int64[grid * 8 * 2], per wave
//     s_memtime at the start and the end of its rounds (0 for idle waves);
//     dig: device int32[grid * 8].  Returns 0, 1 for a bad argument, 2 for a
//     launch error.
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

// Issue-rate probe (see the C ABI note at the top).  The vector instructions
// are written as inline asm so the compiler neither merges nor reorders
// them; each result is read again only rounds later.
template <int KIND>
__global__ __launch_bounds__(512) void k_issue(int iters, int wps, long long *__restrict__ cyc,
                                               int *__restrict__ dig) {
  const int tid = threadIdx.x, w = tid >> 6;
  const int slot = blockIdx.x * 8 + w;
  if (w >= 4 * wps) {
    if ((tid & 63) == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cyc[slot * 4 + e] = 0;
      dig[slot] = 0;
    }
    return;
  }
  float a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0.25f + 0.01f * (float)i + 1e-4f * (float)(tid & 63);
    b[i] = -a[i];
  }
  const uint32_t u = 0x3C803C80u + (uint32_t)(tid & 3);
  const v8bf x = __builtin_bit_cast(v8bf, v4i{(int)u, (int)u, (int)(u ^ 1u), (int)u});
  v4f c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = v4f{(float)i, 0.f, 0.f, 0.f};
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0) {
        asm volatile("v_fma_f32 %0, %1, %1, %0" : "+v"(b[i]) : "v"(a[i]));
      } else if constexpr (KIND == 1) {
        asm volatile("v_exp_f32 %0, %1" : "=v"(b[i]) : "v"(a[i]));
      } else {
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, x, c[i], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KIND == 3) {
          asm volatile("v_fma_f32 %0, %1, %1, %0" : "+v"(b[i]) : "v"(a[i]));
          asm volatile("v_fma_f32 %0, %1, %1, %0" : "+v"(a[(i + 4) & 7]) : "v"(b[(i + 2) & 7]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  int d = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    d = d * 3 + __builtin_bit_cast(int, a[i] + b[i]) + __builtin_bit_cast(int, c[i][0] + c[i][3]);
  if ((tid & 63) == 0) {
    cyc[slot * 4 + 0] = t0;
    cyc[slot * 4 + 1] = t1;
    cyc[slot * 4 + 2] = r0;
    cyc[slot * 4 + 3] = r1;
    dig[slot] = d;
  }
}

// Operand-delivery probe (see the C ABI note at the top).  The piece index
// passes through an empty asm every round so the reads cannot be hoisted.
template <int KIND>
__global__ __launch_bounds__(512) void k_stream(int iters, int waves, const v4i *__restrict__ buf,
                                                long long *__restrict__ cyc, int *__restrict__ dig) {
  __shared__ v4i lds[1024];  // 16 KiB
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int slot = blockIdx.x * 8 + w;
  if constexpr (KIND == 1) {
    for (int i = tid; i < 1024; i += 512) lds[i] = v4i{i, i ^ 1, i ^ 2, i ^ 3};
    __syncthreads();
  }
  if (w >= waves) {
    if (lane == 0) {
      cyc[slot * 2] = 0;
      cyc[slot * 2 + 1] = 0;
      dig[slot] = 0;
    }
    return;
  }
  const v4i *g = buf + (size_t)blockIdx.x * 1024;
  v4i acc = {0, 0, 0, 0};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    int base = (it & 1) * 512;
    asm volatile("" : "+v"(base));
    v4i x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = KIND == 0 ? g[base + i * 64 + lane] : lds[base + i * 64 + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= x[i];
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    cyc[slot * 2] = t0;
    cyc[slot * 2 + 1] = t1;
  }
  if (lane == 0) dig[slot] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace slapeak

extern "C" int slapeak_stream(int kind, int waves, int iters, int grid, const void *buf,
                              long long *cyc, int *dig, hipStream_t st) {
  using namespace slapeak;
  if (kind < 0 || kind > 1 || waves < 1 || waves > 8 || iters < 1 || grid < 1 || !cyc || !dig ||
      (kind == 0 && !buf))
    return 1;
  if (kind == 0)
    k_stream<0><<<grid, 512, 0, st>>>(iters, waves, (const v4i *)buf, cyc, dig);
  else
    k_stream<1><<<grid, 512, 0, st>>>(iters, waves, (const v4i *)buf, cyc, dig);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int slapeak_issue(int kind, int wps, int iters, int grid, long long *cyc, int *dig,
                             hipStream_t st) {
  using namespace slapeak;
  if (kind < 0 || kind > 3 || wps < 1 || wps > 2 || iters < 1 || grid < 1 || !cyc || !dig) return 1;
  switch (kind) {
    case 0: k_issue<0><<<grid, 512, 0, st>>>(iters, wps, cyc, dig); break;
    case 1: k_issue<1><<<grid, 512, 0, st>>>(iters, wps, cyc, dig); break;
    case 2: k_issue<2><<<grid, 512, 0, st>>>(iters, wps, cyc, dig); break;
    default: k_issue<3><<<grid, 512, 0, st>>>(iters, wps, cyc, dig); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

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
