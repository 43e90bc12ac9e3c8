// Decode attention for gfx950: one new query row per (batch entry, head)
// attending a long key/value cache, o = softmax(scale q K^T) V.
//
// This is the generation loop of the pages (a decoder emitting one token at a
// time, each step attending all earlier positions: muhitai.com, "What Is
// Masked Attention?"; notebook chapter, "Masked Attention in the Decoder").
// With one query row the work is 4 d flops per 4 d bytes of K/V: bound by HBM,
// not by the matrix cores, so it runs on the vector ALUs and is organised
// around the memory stream:
//
//   * attn_decode_split_kernel: one work-group per (b*h, key chunk of
//     keys_per_split); each wave streams its contiguous quarter of the chunk
//     with 16-byte loads straight into registers (a 1 KB load covers 4 rows at
//     d = 128, 8 at d = 64; eight K and eight V loads in flight per wave).
//     Lane (slot, c) holds chunk c (8 elements) of one row; the row's score is
//     its 8-element dot product summed over the row's lanes with DPP, so every
//     lane of the row ends with the full score.  Each lane keeps its own
//     running (max, sum, 8 output elements) over the rows it saw; the lanes of
//     a wave and then the four waves merge their states at the end, and the
//     work-group writes one partial (max, sum, d unnormalised outputs).
//   * attn_decode_merge_kernel: one work-group per b*h combines the partials
//     with the same rescaling, divides, rounds once to bf16.
//
// Scores are kept in log2 units (the fp32 dot product times |scale| log2(e));
// the weights exp2(s - m) stay fp32 (no bf16 rounding before the weighted sum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecLoads = 8;          // 1 KB loads of K (and of V) per wave per iteration
constexpr int kDecMaxWg = 8192;       // split work-groups the key chunk size aims to stay under

// DPP row operations (gfx9 encodings): quad_perm [1,0,3,2], [2,3,0,1];
// row_half_mirror (lane i <- 7 - i within 8); row_mirror (i <- 15 - i within 16)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// sum over the CPR consecutive lanes that hold one row (CPR = 8 or 16), in every lane
template <int CPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  if constexpr (CPR == 16) x += dpp<0x140>(x);
  return x;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// combine two (max, sum, acc) states in place; max = -inf means empty
__device__ __forceinline__ void merge_state(float& m, float& l, float (&acc)[8], float m2, float l2,
                                            const float (&acc2)[8]) {
  const float mm = fmaxf(m, m2);
  const float mu = mm == -__builtin_inff() ? 0.f : mm;
  const float f1 = __builtin_amdgcn_exp2f(m - mu), f2 = __builtin_amdgcn_exp2f(m2 - mu);
  l = l * f1 + l2 * f2;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] * f1 + acc2[e] * f2;
  m = mm;
}

template <int D, bool KEYPAD>
__global__ __launch_bounds__(kDecThreads) void attn_decode_split_kernel(DecParams p) {
  constexpr int ROWB = D * 2;            // bytes per row
  constexpr int CPR = D / 8;             // lanes per row (16 bytes each)
  constexpr int RPL = 64 / CPR;          // rows per 1 KB wave load
  constexpr int RPI = RPL * kDecLoads;   // rows per wave iteration
  constexpr float kNegInf = -__builtin_inff();

  __shared__ float sm_acc[kDecWaves][D];
  __shared__ float sm_ml[kDecWaves][2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane % CPR, slot = lane / CPR;
  const int bh = blockIdx.x / p.n_split, sp = blockIdx.x - bh * p.n_split;
  const int b = bh / p.H;
  int L = p.Tk;
  if (KEYPAD) L = clamp_len(p.key_lens, b, p.Tk);
  const int per_wave = p.keys_per_split / kDecWaves;
  const int r0 = sp * p.keys_per_split + w * per_wave;
  const int r1 = min(r0 + per_wave, L);

  // this lane's 8 query elements (negated for a negative scale: exact)
  float qf[8];
  {
    u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.q) + (int64_t)bh * D + 8 * c);
    if (p.neg) x ^= 0x80008000u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf_lo(x[i]);
      qf[2 * i + 1] = bf_hi(x[i]);
    }
  }
  const float cs = p.scale_log2;
  float m = kNegInf, l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  if (r0 < r1) {
    const int64_t head = (int64_t)bh * p.Tk * D;
    // the descriptors cover rows [0, L) of this head: rows past L read as 0
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(static_cast<const __bf16*>(p.k) + head, (uint32_t)L * ROWB);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(static_cast<const __bf16*>(p.v) + head, (uint32_t)L * ROWB);
    for (int rb = r0; rb < r1; rb += RPI) {
      u32x4 kx[kDecLoads], vx[kDecLoads];
#pragma unroll
      for (int u = 0; u < kDecLoads; ++u) {
        // each cache row is read once: non-temporal loads (aux bit 1, "nt")
        // keep the stream from displacing cached data and read faster
        // (a plain read of 1 GiB: 6.3-6.5 TB/s, non-temporal: 7.0 TB/s)
        const uint32_t off = (uint32_t)(rb + u * RPL + slot) * ROWB + 16 * c;
        kx[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 2));
        vx[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 2));
      }
      float s[kDecLoads];
      float mt = m;
#pragma unroll
      for (int u = 0; u < kDecLoads; ++u) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          part = __builtin_fmaf(qf[2 * i], bf_lo(kx[u][i]), part);
          part = __builtin_fmaf(qf[2 * i + 1], bf_hi(kx[u][i]), part);
        }
        const float sc = row_sum<CPR>(part) * cs;
        s[u] = (rb + u * RPL + slot < r1) ? sc : kNegInf;
        mt = fmaxf(mt, s[u]);
      }
      const float mu = mt == kNegInf ? 0.f : mt;
      const float f = __builtin_amdgcn_exp2f(m - mu);
      l *= f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= f;
      m = mt;
#pragma unroll
      for (int u = 0; u < kDecLoads; ++u) {
        const float pu = __builtin_amdgcn_exp2f(s[u] - mu);
        l += pu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(pu, bf_lo(vx[u][i]), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(pu, bf_hi(vx[u][i]), acc[2 * i + 1]);
        }
      }
    }
  }

  // merge the row slots of the wave (lanes c, c + CPR, ...)
#pragma unroll
  for (int x = CPR; x < 64; x <<= 1) {
    float acc2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc2[e] = __shfl_xor(acc[e], x, 64);
    const float m2 = __shfl_xor(m, x, 64), l2 = __shfl_xor(l, x, 64);
    merge_state(m, l, acc, m2, l2, acc2);
  }
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_acc[w][8 * c + e] = acc[e];
    if (c == 0) {
      sm_ml[w][0] = m;
      sm_ml[w][1] = l;
    }
  }
  __syncthreads();
  if (tid < D) {
    float mm = kNegInf;
#pragma unroll
    for (int i = 0; i < kDecWaves; ++i) mm = fmaxf(mm, sm_ml[i][0]);
    const float mu = mm == kNegInf ? 0.f : mm;
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int i = 0; i < kDecWaves; ++i) {
      const float f = __builtin_amdgcn_exp2f(sm_ml[i][0] - mu);
      o += f * sm_acc[i][tid];
      ls += f * sm_ml[i][1];
    }
    const int64_t part = (int64_t)bh * p.n_split + sp;
    p.part_acc[part * D + tid] = o;
    if (tid == 0) {
      p.part_ml[2 * part] = mm;
      p.part_ml[2 * part + 1] = ls;
    }
  }
}

// One work-group (one lane per output element) per (b, head).  The splits'
// maxima are read and reduced in parallel; then, chunk by chunk, each lane
// computes one split's weight exp2(m_s - M) into LDS and every lane sums its
// element over the chunk with independent loads.
template <int D>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(DecParams p) {
  constexpr float kNegInf = -__builtin_inff();
  constexpr int NW = D / 64;
  __shared__ float sf[D], sl[D], sred[NW];
  const int bh = blockIdx.x, t = threadIdx.x;
  const int ns = p.n_split;
  const float* ml = p.part_ml + (int64_t)bh * ns * 2;
  const float* pa = p.part_acc + (int64_t)bh * ns * D;
  float mm = kNegInf;
  for (int s = t; s < ns; s += D) mm = fmaxf(mm, ml[2 * s]);
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) mm = fmaxf(mm, __shfl_xor(mm, x, 64));
  if ((t & 63) == 0) sred[t >> 6] = mm;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) mm = fmaxf(mm, sred[i]);
  const float mu = mm == kNegInf ? 0.f : mm;
  float o = 0.f, ls = 0.f;
  for (int s0 = 0; s0 < ns; s0 += D) {
    float f = 0.f, lw = 0.f;
    if (s0 + t < ns) {
      f = __builtin_amdgcn_exp2f(ml[2 * (s0 + t)] - mu);
      lw = f * ml[2 * (s0 + t) + 1];
    }
    sf[t] = f;
    sl[t] = lw;
    __syncthreads();
    const int n = min(D, ns - s0);
    const float* src = pa + (int64_t)s0 * D + t;
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      o += sf[j] * src[(int64_t)j * D];
      ls += sl[j];
    }
    __syncthreads();
  }
  static_cast<__bf16*>(p.o)[(int64_t)bh * D + t] = (__bf16)(ls > 0.f ? o / ls : 0.f);
}

// ---------------------------------------------------------------------------

int decode_keys_per_split(int B, int H, int Tk) {
  const int64_t bh = (int64_t)B * H;
  int64_t kps = 256;
  while (kps < Tk && bh * ((Tk + kps - 1) / kps) > kDecMaxWg) kps *= 2;
  return (int)kps;
}

int decode_splits(int B, int H, int Tk) {
  const int kps = decode_keys_per_split(B, H, Tk);
  return Tk > 0 ? (Tk + kps - 1) / kps : 1;
}

template <int D>
static hipError_t launch_decode_d(const DecParams& prm, bool keypad, hipStream_t stream) {
  DecParams local = prm;
  void* args[] = {&local};
  const void* split = keypad ? reinterpret_cast<const void*>(&attn_decode_split_kernel<D, true>)
                             : reinterpret_cast<const void*>(&attn_decode_split_kernel<D, false>);
  hipError_t e = hipLaunchKernel(split, dim3(prm.B * prm.H * prm.n_split), dim3(kDecThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_decode_merge_kernel<D>), dim3(prm.B * prm.H),
                         dim3(D), args, 0, stream);
}

hipError_t launch_decode(const DecParams& prm, int d, bool keypad, hipStream_t stream) {
  return d == 64 ? launch_decode_d<64>(prm, keypad, stream) : launch_decode_d<128>(prm, keypad, stream);
}

}  // namespace attn
