// Backward pass of scaled dot-product attention for gfx950 (MI355X):
// gradients of O = softmax(scale * Q K^T) V with respect to Q, K and V, bf16
// in and out, fp32 accumulation.
//
// With P the row-softmax weights (recomputed as exp(scale s - lse) from the
// forward's log-sum-exp), dO the incoming gradient and D_i = dO_i . O_i:
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q
// (chain rule through O = P V and the row softmax; training through the
// formula is what the pages describe: aiany.app Step 11, cross-entropy
// training of every weight matrix).
//
// Two kernels, no atomics and no scratch beyond the caller's delta array:
//   * attn_bwd_dq_kernel: one work-group per 128 query rows (d = 64) or 256
//     (d = 128); writes D_i and lse_i log2(e) to the caller's workspace, then
//     streams K/V tiles of 64 keys and accumulates dQ in registers;
//   * attn_bwd_dkdv_kernel: one work-group per 128 keys (d = 64) or 256 keys
//     (d = 128: 8 waves, V's rows held in LDS so two waves fit on a SIMD);
//     streams Q/dO tiles of 64 rows (with their D and lse log2(e)) and
//     accumulates dK, dV in registers.
// Matrix-core mapping as in the forward (v_mfma_f32_32x32x16_bf16, lane l,
// g = l / 32, c = l % 32): products whose output rows are the lane's own
// row/key take the streamed operand from LDS as 16-byte fragments read in
// slot order sigma; products contracting over the streamed index take it
// transposed with ds_read_b64_tr_b16.  Both read patterns share one tile
// layout that is free of bank conflicts for both: an XOR swizzle of the
// chunks (dual_swz) with per-step offsets in registers, or, in the d = 128
// dK/dV kernel, padded 288-byte row slots whose per-step offsets are
// constants on one base (PadTile128).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

// A test-only build (-DATTN_BWD_TEST_SERIAL_STAGING=1, built as
// libattn_serial_test.so, never as libattn.so) waits for each step's
// direct-to-LDS loads before the step reads LDS, in the dQ, dK/dV and weights
// kernels: no load is in flight while any wave reads a tile, so the staging
// cannot race; their outputs must equal the pipelined kernels' bit for bit.
#ifndef ATTN_BWD_TEST_SERIAL_STAGING
#define ATTN_BWD_TEST_SERIAL_STAGING 0
#endif

namespace attn {

constexpr bool kBwdSerialStaging = ATTN_BWD_TEST_SERIAL_STAGING != 0;

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBT = 64;            // keys (dQ kernel) or query rows (dK/dV kernel) per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BwdTile {
  static constexpr int ROWB = D * 2;                       // bytes per row
  static constexpr int TILEB = kBT * ROWB;                 // bytes per tile
  static constexpr int NLD = TILEB / 1024 / kBwdWaves;     // 1 KB direct loads per wave
  static constexpr int DT = D / 16;                        // MFMA steps over d
  static constexpr int NO = D / 32;                        // 32-column output tiles
};

// direct-to-LDS source offsets of this lane for a row-major 64-row tile,
// stored with the dual swizzle
template <int D, int W = kBwdWaves>
__device__ __forceinline__ void tile_src_offsets(int w, int lane, uint32_t (&src)[BwdTile<D>::TILEB / 1024 / W]) {
  constexpr int ROWB = BwdTile<D>::ROWB;
#pragma unroll
  for (int u = 0; u < BwdTile<D>::TILEB / 1024 / W; ++u) {
    const int pos = (W * u + w) * 1024 + 16 * lane;
    const int r = pos / ROWB, pc = (pos % ROWB) / 16;
    src[u] = r * ROWB + 16 * (pc ^ dual_swz<D>(r));
  }
}

// fragment-read offsets: lane (c, g), step t reads logical chunk 2t + g of row
// sigma(c) (+ 32 hh rows, an immediate): the A operand of a product whose
// output rows follow the S^T / S slot order
template <int D>
__device__ __forceinline__ void frag_offsets(int c, int g, int (&rd)[BwdTile<D>::DT]) {
  const int r = sigma32(c);
#pragma unroll
  for (int t = 0; t < BwdTile<D>::DT; ++t) rd[t] = r * BwdTile<D>::ROWB + 16 * ((2 * t + g) ^ dual_swz<D>(r));
}

// transposed-read offsets: in 16-lane group G (h = G & 1, gg = G >> 1) source
// lane s reads 4 consecutive output columns of row 8gg + 4e + s/4 (+ 16m rows,
// an immediate); index [i][e] for output tile i and row half e
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&rd)[BwdTile<D>::NO][2]) {
  const int G = lane >> 4, sl = lane & 15;
  const int h = G & 1, gg = G >> 1;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 8 * gg + 4 * e + (sl >> 2);
#pragma unroll
    for (int i = 0; i < BwdTile<D>::NO; ++i) {
      const int lc = (D / 16) * (sl & 1) + 2 * i + h;
      rd[i][e] = r * BwdTile<D>::ROWB + 16 * (lc ^ dual_swz<D>(r)) + 8 * ((sl >> 1) & 1);
    }
  }
}

// A operand (8 consecutive rows of the transposed tile) from two transposed reads
__device__ __forceinline__ bf16x8 tr_fragment(const char* lo_addr, const char* hi_addr) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lo_addr));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(hi_addr));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// lane's row of a bf16 [., D] matrix in the B-operand layout (d = 16t + 8g + e)
template <int D>
__device__ __forceinline__ void load_row(const __bf16* base, int row, int nrows, int g, bool negate,
                                         bf16x8 (&f)[BwdTile<D>::DT]) {
  const bool ok = row < nrows;
  const __bf16* rp = base + (int64_t)(ok ? row : 0) * D + 8 * g;
#pragma unroll
  for (int t = 0; t < BwdTile<D>::DT; ++t) {
    u32x4 x = ok ? *reinterpret_cast<const u32x4*>(rp + 16 * t) : u32x4{0, 0, 0, 0};
    if (negate) x ^= 0x80008000u;
    f[t] = __builtin_bit_cast(bf16x8, x);
  }
}

// store a lane's accumulated row (columns tau: (D/2) g + 16 i + r) times `mul`
template <int D>
__device__ __forceinline__ void store_row(__bf16* base, int row, int g, float mul,
                                          const f32x16 (&acc)[BwdTile<D>::NO]) {
  __bf16* op = base + (int64_t)row * D + (D / 2) * g;
#pragma unroll
  for (int i = 0; i < BwdTile<D>::NO; ++i)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x8 o8;
#pragma unroll
      for (int j = 0; j < 8; ++j) o8[j] = acc[i][8 * h2 + j] * mul;
      *reinterpret_cast<bf16x8*>(op + 16 * i + 8 * h2) = __builtin_convertvector(o8, bf16x8);
    }
}

// ---------------------------------------------------------------------------
// dQ (and D) kernel
// ---------------------------------------------------------------------------
// dQ work-group shape: d = 128 runs 8 waves (256 rows, two waves per SIMD), so
// each K/V tile staged in LDS serves twice as many rows; d = 64 runs 4
template <int D>
struct DqShape {
  static constexpr int kWaves = D == 128 ? 8 : kBwdWaves;
};

template <int D, bool CAUSAL, bool KEYPAD>
__global__ __launch_bounds__(64 * DqShape<D>::kWaves, 8 / DqShape<D>::kWaves) void attn_bwd_dq_kernel(BwdParams p) {
  using TG = BwdTile<D>;
  constexpr int W = DqShape<D>::kWaves;
  constexpr int ROWB = TG::ROWB, TILEB = TG::TILEB, DT = TG::DT, NO = TG::NO;
  constexpr int NLD = TILEB / 1024 / W;
  constexpr int BM = 32 * W;
  constexpr float kNegInf = -__builtin_inff(), kPosInf = __builtin_inff();

  __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb1[TILEB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  int bh, qt;
  tile_of_block(p.n_qtiles, CAUSAL, bh, qt);
  const int b = bh / p.H;
  const int Tq = p.Tq, Tk = p.Tk;
  const int q0 = qt * BM, qw = q0 + 32 * w, row = qw + c;
  int kend = Tk;
  if (KEYPAD) kend = min(kend, clamp_len(p.key_lens, b, Tk));
  int kend_wg = CAUSAL ? min(kend, q0 + BM) : kend;
  const int ntiles = kend_wg > 0 ? (kend_wg + kBT - 1) / kBT : 0;
  int kend_w = CAUSAL ? min(kend, qw + 32) : kend;
  if (qw >= Tq) kend_w = 0;
  const int ntw = kend_w > 0 ? (kend_w + kBT - 1) / kBT : 0;

  const int64_t qoff = (int64_t)bh * Tq * D, koff = (int64_t)bh * Tk * D;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + koff;
  const __bf16* Vg = static_cast<const __bf16*>(p.v) + koff;

  bf16x8 qf[DT], gf[DT];
  load_row<D>(static_cast<const __bf16*>(p.q) + qoff, row, Tq, g, p.neg != 0, qf);
  load_row<D>(static_cast<const __bf16*>(p.dout) + qoff, row, Tq, g, false, gf);
  // D_i = dO_i . O_i (each lane half holds d/2 of the products)
  float delta;
  {
    bf16x8 of[DT];
    load_row<D>(static_cast<const __bf16*>(p.o) + qoff, row, Tq, g, false, of);
    float part = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) part += (float)gf[t][e] * (float)of[t][e];
    delta = pair_sum(part);
  }
  float l2 = kPosInf;   // lse in log2 units; +inf makes every weight of an empty row 0
  if (row < Tq) {
    const float lse = p.lse[(int64_t)bh * Tq + row];
    l2 = lse == kNegInf ? kPosInf : lse * kLog2e;
    if (g == 0) {
      p.delta[(int64_t)bh * Tq + row] = delta;
      p.delta[(int64_t)p.B * p.H * Tq + (int64_t)bh * Tq + row] = l2;
    }
  }

  uint32_t src[NLD];
  tile_src_offsets<D, W>(w, lane, src);
  auto load_kv = [&](int j0, char* kt, char* vt) __attribute__((always_inline)) {
    const uint32_t bytes = (uint32_t)(kend - j0) * ROWB;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (int64_t)j0 * D, bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (int64_t)j0 * D, bytes);
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      lds_dma16(kr, kt + (W * u + w) * 1024, src[u]);
      lds_dma16(vr, vt + (W * u + w) * 1024, src[u]);
    }
  };
  int fr[DT];
  frag_offsets<D>(c, g, fr);
  int trd[NO][2];
  tr_offsets<D>(lane, trd);

  f32x16 acc[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) acc[i] = f32x16{};
  const float cs = p.scale_log2;

  auto step = [&](int it, const char* kt, const char* vt) __attribute__((always_inline)) {
    const int j0 = it * kBT;
    const bool edge = (j0 + kBT > kend) || (CAUSAL && j0 + kBT - 1 > qw);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + 32 * hh * ROWB + fr[t]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s, 0, 0, 0);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vt + 32 * hh * ROWB + fr[t]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, gf[t], dp, 0, 0, 0);
      }
      // register e: key j0 + 32hh + 16(e/8) + 8g + e%8 of this lane's row
      f32x16 pr;
#pragma unroll
      for (int e = 0; e < 16; ++e) pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], cs, -l2));
      if (edge) {   // one wave-uniform branch: allowed keys of this row are [0, hi)
        const int hi = CAUSAL ? min(kend, row + 1) : kend;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j0 + 32 * hh + 16 * (e >> 3) + 8 * g + (e & 7);
          pr[e] = key < hi ? pr[e] : 0.f;
        }
      }
      f32x16 ds;
#pragma unroll
      for (int e = 0; e < 16; ++e) ds[e] = pr[e] * (dp[e] - delta);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x8 d8;
#pragma unroll
        for (int j = 0; j < 8; ++j) d8[j] = ds[8 * m + j];
        const bf16x8 dsb = __builtin_convertvector(d8, bf16x8);
        const char* kb = kt + (32 * hh + 16 * m) * ROWB;
#pragma unroll
        for (int i = 0; i < NO; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_fragment(kb + trd[i][0], kb + trd[i][1]), dsb,
                                                           acc[i], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) load_kv(0, kb0, vb0);
  pipeline_barrier<0>();
  for (int it0 = 0; it0 < ntiles; it0 += 2) {
    static_for<0, 2>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      const int it = it0 + u;
      if (it < ntiles) {
        if (it + 1 < ntiles) load_kv((it + 1) * kBT, u ? kb0 : kb1, u ? vb0 : vb1);
        if constexpr (kBwdSerialStaging) pipeline_barrier<0>();   // test build only
        if (it < ntw) step(it, u ? kb1 : kb0, u ? vb1 : vb0);
        pipeline_barrier<0>();
      }
    });
  }
  if (row < Tq) store_row<D>(static_cast<__bf16*>(p.dq) + qoff, row, g, p.scale, acc);
}

// ---------------------------------------------------------------------------
// dK / dV kernel
// ---------------------------------------------------------------------------
// dK/dV work-group shape: d = 128 runs 8 waves (two per SIMD, 256 keys) with
// V's rows in LDS, so a wave holds only its K row and the accumulators; d = 64
// fits 4 waves with K and V in registers
template <int D>
struct DkdvShape {
  static constexpr int kWaves = D == 128 ? 8 : kBwdWaves;
  static constexpr bool kVInLds = D == 128;
};

// Q / dO tiles of the d = 128 dK/dV kernel: 64 rows of 256 bytes, row r at
// byte 288 r + 16 ((r >> 3) & 1) of the tile (a 288-byte slot per row, the row
// shifted by 16 bytes when bit 3 of r is set).  Both read patterns are free of
// bank conflicts -- 16-byte fragments of 16 rows in sigma order (16 distinct
// 16-byte bank groups) and transposed reads of 4 consecutive rows at two chunk
// columns 128 bytes apart (32 distinct 8-byte groups) -- and, unlike an XOR
// swizzle, the offset of every step is a constant added to one per-lane base,
// so the reads cost no address arithmetic.  The 32 spare bytes per row are
// filled by loads past the buffer's range (zeros, no memory access).
struct PadTile128 {
  static constexpr int SLOT = 288;
  static constexpr int BYTES = 64 * SLOT;        // 18 KB
  static constexpr int UNITS = BYTES / 1024;     // 1 KB direct-to-LDS loads per tile
  __device__ static constexpr int row(int r) { return SLOT * r + 16 * ((r >> 3) & 1); }
  // source offset (row-major 256-byte rows) of the 16 bytes at tile byte pos, or pad for a gap
  __device__ static uint32_t src(int pos, uint32_t pad) {
    const int r = pos / SLOT, k = pos - row(r);
    return (k >= 0 && k < 256) ? (uint32_t)(r * 256 + k) : pad;
  }
};
// V rows of the d = 128 dK/dV work-group (256 keys): row r at byte 272 r; each
// lane reads only its own key's row, 16 consecutive rows per 16 lanes, which
// the 272-byte stride spreads over all 64 banks
constexpr int kVRowSlot = 272;

// launder a value through an empty asm: the compiler can no longer split a
// constant out of it, so base + small constant stays one LDS offset field
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, bool CAUSAL, bool KEYPAD>
__global__ __launch_bounds__(64 * DkdvShape<D>::kWaves, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  using TG = BwdTile<D>;
  constexpr int W = DkdvShape<D>::kWaves;
  constexpr bool VLDS = DkdvShape<D>::kVInLds;
  static_assert(!VLDS || D == 128, "the padded layout is laid out for d = 128");
  constexpr int ROWB = TG::ROWB, DT = TG::DT, NO = TG::NO;
  constexpr int BK = 32 * W;
  // LDS block: Q tile 0, Q tile 1, dO tile 0, dO tile 1, (d = 128) the V rows,
  // then per tile the lse * log2(e) of its 64 rows in [0, 64) and D in [64, 128)
  constexpr int TB = VLDS ? PadTile128::BYTES : TG::TILEB;
  constexpr int NLD = VLDS ? (PadTile128::UNITS + W - 1) / W : TG::TILEB / 1024 / W;
  constexpr int VROWSB = VLDS ? BK * kVRowSlot : 0;
  constexpr int VUNITS = VROWSB / 1024;
  static_assert(VROWSB % 1024 == 0 && NLD >= 1, "tile shape");
  constexpr int RB = 4 * TB + VROWSB;   // lse / D of tile u at RB + 512 u
  __shared__ __attribute__((aligned(1024))) char lds[RB + 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  int bh, kt;
  tile_of_block(p.n_ktiles, false, bh, kt);
  const int b = bh / p.H;
  const int Tq = p.Tq, Tk = p.Tk;
  const int k0 = kt * BK, kw = k0 + 32 * w, key = kw + c;
  int kend = Tk;
  if (KEYPAD) kend = min(kend, clamp_len(p.key_lens, b, Tk));
  const int nq = (Tq + kBT - 1) / kBT;
  const int first = CAUSAL ? min(k0 / kBT, nq) : 0;   // rows below k0 see none of these keys
  const int ntiles = k0 < kend ? nq - first : 0;

  const int64_t qoff = (int64_t)bh * Tq * D, koff = (int64_t)bh * Tk * D;
  const __bf16* Qg = static_cast<const __bf16*>(p.q) + qoff;
  const __bf16* Gg = static_cast<const __bf16*>(p.dout) + qoff;
  const float* Dg = p.delta + (int64_t)bh * Tq;                                  // D
  const float* Lg = p.delta + (int64_t)p.B * p.H * Tq + (int64_t)bh * Tq;       // lse * log2(e)

  // this lane's key row: K negated for a negative scale (S = scale Q K^T), and V
  bf16x8 kf[DT], vf[VLDS ? 1 : DT];
  load_row<D>(static_cast<const __bf16*>(p.k) + koff, key, kend, g, p.neg != 0, kf);
  int vb = 0;
  if constexpr (VLDS) {
    // the work-group's V rows into LDS once (rows at or past kend, and the
    // spare bytes of each slot, read as zero)
    const __bf16* Vb = static_cast<const __bf16*>(p.v) + koff + (int64_t)k0 * D;
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vb, (uint32_t)max(min(kend - k0, BK), 0) * ROWB);
#pragma unroll
    for (int u = 0; u < (VUNITS + W - 1) / W; ++u) {
      const int unit = W * u + w;
      if (unit < VUNITS) {
        const int pos = unit * 1024 + 16 * lane;
        const int r = pos / kVRowSlot, k = pos - r * kVRowSlot;
        lds_dma16(vr, lds + 4 * TB + unit * 1024, k < ROWB ? (uint32_t)(r * ROWB + k) : (uint32_t)(BK * ROWB));
      }
    }
    // chunk 2t + g of row 32w + c: base + 32 t
    vb = opaque(4 * TB + (32 * w + c) * kVRowSlot + 16 * g);
  } else {
    load_row<D>(static_cast<const __bf16*>(p.v) + koff, key, kend, g, false, vf);
  }

  uint32_t src[NLD];
  if constexpr (VLDS) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) src[u] = PadTile128::src((W * u + w) * 1024 + 16 * lane, 64 * ROWB);
  } else {
    tile_src_offsets<D, W>(w, lane, src);
  }
  // tile buffers by index: Q tile u at u * TB, dO tile u at (2 + u) * TB
  auto load_tile = [&](int r0, int u) __attribute__((always_inline)) {
    // the buffer range covers this tile's rows only, so a pad offset of 64 rows is always past it
    const uint32_t bytes = (uint32_t)min(Tq - r0, kBT) * ROWB;
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(Qg + (int64_t)r0 * D, bytes);
    const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(Gg + (int64_t)r0 * D, bytes);
#pragma unroll
    for (int v = 0; v < NLD; ++v) {
      const int unit = W * v + w;
      if (!VLDS || unit < PadTile128::UNITS) {
        lds_dma16(qr, lds + u * TB + unit * 1024, src[v]);
        lds_dma16(gr, lds + (2 + u) * TB + unit * 1024, src[v]);
      }
    }
    // lse * log2(e) (wave 0) and D (wave 1) of rows r0 .. r0 + 63; rows at or past Tq read as 0
    if (w < 2) {
      const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(w == 0 ? Lg + r0 : Dg + r0, (uint32_t)(Tq - r0) * 4);
      lds_dma4(rr, lds + RB + 512 * u + 256 * w, 4 * lane);
    }
  };
  // per-lane read offsets.  d = 128: one base per pattern and tensor, every
  // step a constant on top (fragment: row 32 hh + sigma(c), chunk 2t + g;
  // transposed: row 32 hh + 16 m + 8 gg + 4 e + s / 4, chunk 8 (s & 1) + 2 i + h,
  // half (s >> 1) & 1, for 16-lane group G = 2 gg + h and source lane s); the
  // dO bases carry the dO buffers' offset so their constants stay small.
  // d = 64: the XOR-swizzled offsets of every step held in registers.
  int fr[VLDS ? 1 : DT];
  int trd[VLDS ? 1 : NO][2];
  int fbq = 0, fbg = 0, tbq = 0, tbg = 0;
  if constexpr (VLDS) {
    const int sl = lane & 15, G = lane >> 4, h = G & 1, gg = G >> 1;
    fbq = PadTile128::row(sigma32(c)) + 16 * g;
    tbq = PadTile128::row(8 * gg + (sl >> 2)) + 128 * (sl & 1) + 16 * h + 8 * ((sl >> 1) & 1);
    fbg = opaque(fbq + 2 * TB);
    tbg = opaque(tbq + 2 * TB);
  } else {
    frag_offsets<D>(c, g, fr);
    tr_offsets<D>(lane, trd);
  }
  // Q / dO fragment of row 32 hh + sigma(c), step t, from buffer u
  auto q_frag = [&](int u, int hh, int t) __attribute__((always_inline)) {
    if constexpr (VLDS) return *reinterpret_cast<const bf16x8*>(lds + fbq + u * TB + 32 * PadTile128::SLOT * hh + 32 * t);
    else return *reinterpret_cast<const bf16x8*>(lds + u * TB + 32 * hh * ROWB + fr[t]);
  };
  auto g_frag = [&](int u, int hh, int t) __attribute__((always_inline)) {
    if constexpr (VLDS) return *reinterpret_cast<const bf16x8*>(lds + fbg + u * TB + 32 * PadTile128::SLOT * hh + 32 * t);
    else return *reinterpret_cast<const bf16x8*>(lds + (2 + u) * TB + 32 * hh * ROWB + fr[t]);
  };
  // transposed A operand (8 rows 16 m' .. of the tile at row block rb = 32 hh + 16 m) for output tile i
  auto q_tr = [&](int u, int rb, int i) __attribute__((always_inline)) {
    if constexpr (VLDS) {
      const char* a = lds + tbq + u * TB + PadTile128::SLOT * rb + 32 * i;
      return tr_fragment(a, a + 4 * PadTile128::SLOT);
    } else {
      const char* a = lds + u * TB + rb * ROWB;
      return tr_fragment(a + trd[i][0], a + trd[i][1]);
    }
  };
  auto g_tr = [&](int u, int rb, int i) __attribute__((always_inline)) {
    if constexpr (VLDS) {
      const char* a = lds + tbg + u * TB + PadTile128::SLOT * rb + 32 * i;
      return tr_fragment(a, a + 4 * PadTile128::SLOT);
    } else {
      const char* a = lds + (2 + u) * TB + rb * ROWB;
      return tr_fragment(a + trd[i][0], a + trd[i][1]);
    }
  };

  f32x16 adk[NO], adv[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) adk[i] = adv[i] = f32x16{};
  const float cs = p.scale_log2;

  // lse / D reads: rows 8g .. 8g + 7 of a 16-row group, from one laundered base
  const int rbl = opaque(RB + 32 * g);
  auto step = [&](int it, int u) __attribute__((always_inline)) {
    const char* rt = lds + rbl + 512 * u;
    const int r0 = it * kBT;
    const bool edge = (kw + 32 > kend) || (CAUSAL && r0 < kw + 31) || (r0 + kBT > Tq);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_frag(u, hh, t), kf[t], s, 0, 0, 0);
        const bf16x8 ga = g_frag(u, hh, t);
        bf16x8 vt;
        if constexpr (VLDS) vt = *reinterpret_cast<const bf16x8*>(lds + vb + 32 * t);
        else vt = vf[t];
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, vt, dp, 0, 0, 0);
      }
      // register e: row r0 + 32hh + 16(e/8) + 8g + e%8 for this lane's key
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int rl = 32 * hh + 16 * m + 8 * g;   // first of the 8 rows (tile-local)
        const int ro = 4 * (32 * hh + 16 * m);        // byte offset of the 16-row group
        const f32x4 la = *reinterpret_cast<const f32x4*>(rt + ro);
        const f32x4 lb = *reinterpret_cast<const f32x4*>(rt + ro + 16);
        const f32x4 da = *reinterpret_cast<const f32x4*>(rt + 256 + ro);
        const f32x4 db = *reinterpret_cast<const f32x4*>(rt + 256 + ro + 16);
        f32x8 p8, d8;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float l2 = j < 4 ? la[j] : lb[j - 4];
          const float dlt = j < 4 ? da[j] : db[j - 4];
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * m + j], cs, -l2));
          p8[j] = pe;
          d8[j] = pe * (dp[8 * m + j] - dlt);
        }
        // one wave-uniform branch for the 8 rows; select, not multiply: a masked
        // weight may be inf before it
        if (edge) {
          // valid rows of this lane's key: [lo, hi) (empty for a key past the length)
          const int lo = CAUSAL ? key : 0, hi = key < kend ? Tq : 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int rw = r0 + rl + j;
            const bool ok = rw >= lo && rw < hi;
            p8[j] = ok ? p8[j] : 0.f;
            d8[j] = ok ? d8[j] : 0.f;
          }
        }
        const bf16x8 pb = __builtin_convertvector(p8, bf16x8);
        const bf16x8 dsb = __builtin_convertvector(d8, bf16x8);
#pragma unroll
        for (int i = 0; i < NO; ++i) {
          adv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g_tr(u, 32 * hh + 16 * m, i), pb, adv[i], 0, 0, 0);
          adk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q_tr(u, 32 * hh + 16 * m, i), dsb, adk[i], 0, 0, 0);
        }
      }
    }
  };

  if (ntiles > 0) load_tile(first * kBT, 0);
  pipeline_barrier<0>();
  // pairs of tiles with no condition around the accumulating steps (a
  // conditional step makes the compiler shuttle dK and dV between register
  // files at every trip), then the odd last tile
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    load_tile((first + it + 1) * kBT, 1);
    if constexpr (kBwdSerialStaging) pipeline_barrier<0>();   // test build only
    step(first + it, 0);
    pipeline_barrier<0>();
    if (it + 2 < ntiles) load_tile((first + it + 2) * kBT, 0);
    if constexpr (kBwdSerialStaging) pipeline_barrier<0>();   // test build only
    step(first + it + 1, 1);
    pipeline_barrier<0>();
  }
  if (it < ntiles) step(first + it, 0);
  if (key < Tk) {
    store_row<D>(static_cast<__bf16*>(p.dk) + koff, key, g, p.scale, adk);
    store_row<D>(static_cast<__bf16*>(p.dv) + koff, key, g, 1.0f, adv);
  }
}

// ---------------------------------------------------------------------------
// Attention weights output: w_ij = exp(scale s_ij - lse_i), masked entries 0,
// the whole [Tq, Tk] matrix of every (b, head) written as fp32.  One
// work-group per 128 query rows walks all key tiles of 64: tiles inside the
// causal / padding limit recompute S^T = K Q^T on the matrix cores (K tiles
// double-buffered in LDS as in the dQ kernel), tiles past it are written as
// zeros without loading anything.  The weights leave the registers through a
// per-wave 32 x 32 fp32 LDS block (row r's 16-byte chunk k at chunk k ^ (r/2)
// of a 128-byte row: conflict-free for the 16-byte writes of the MFMA layout
// and for the row-wise reads), so every global store instruction writes 8
// whole 128-byte row segments; scalar stores when Tk is not a multiple of 4 or
// at the ragged end.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool KEYPAD>
__global__ __launch_bounds__(kBwdThreads, 2) void attn_weights_kernel(WtsParams p) {
  using TG = BwdTile<D>;
  constexpr int ROWB = TG::ROWB, TILEB = TG::TILEB, NLD = TG::NLD, DT = TG::DT;
  constexpr int BM = 32 * kBwdWaves;
  constexpr float kNegInf = -__builtin_inff(), kPosInf = __builtin_inff();

  __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
  __shared__ __attribute__((aligned(1024))) float stage[kBwdWaves][32 * 32];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  int bh, qt;
  tile_of_block(p.n_qtiles, CAUSAL, bh, qt);
  const int b = bh / p.H;
  const int Tq = p.Tq, Tk = p.Tk;
  const int q0 = qt * BM, qw = q0 + 32 * w, row = qw + c;
  int kend = Tk;
  if (KEYPAD) kend = min(kend, clamp_len(p.key_lens, b, Tk));
  const int kend_wg = CAUSAL ? min(kend, q0 + BM) : kend;
  const int ntiles = kend_wg > 0 ? (kend_wg + kBT - 1) / kBT : 0;       // tiles with any allowed key
  const int nall = (Tk + kBT - 1) / kBT;                                // tiles to write

  const int64_t qoff = (int64_t)bh * Tq * D, koff = (int64_t)bh * Tk * D;
  const __bf16* Kg = static_cast<const __bf16*>(p.k) + koff;
  bf16x8 qf[DT];
  load_row<D>(static_cast<const __bf16*>(p.q) + qoff, row, Tq, g, p.neg != 0, qf);
  float l2 = kPosInf;
  if (row < Tq) {
    const float lse = p.lse[(int64_t)bh * Tq + row];
    l2 = lse == kNegInf ? kPosInf : lse * kLog2e;
  }
  const bool vec = (Tk & 3) == 0;
  float* const wbh = p.w + (int64_t)bh * Tq * Tk;
  float* const st = stage[w];
  // row-wise store pattern: lane writes 4 keys (16 bytes) at chunk sc of rows sr + 8 i
  const int sr = lane >> 3, sc = lane & 7;

  uint32_t src[NLD];
  tile_src_offsets<D>(w, lane, src);
  auto load_k = [&](int j0, char* kt) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (int64_t)j0 * D, (uint32_t)(kend - j0) * ROWB);
#pragma unroll
    for (int u = 0; u < NLD; ++u) lds_dma16(kr, kt + (kBwdWaves * u + w) * 1024, src[u]);
  };
  int fr[DT];
  frag_offsets<D>(c, g, fr);
  const float cs = p.scale_log2;

  // 4 keys j .. j+3 of query row r (wave-relative) to global memory
  auto store4 = [&](int r, int j, const f32x4& v4) __attribute__((always_inline)) {
    if (qw + r >= Tq) return;
    float* dst = wbh + (int64_t)(qw + r) * Tk + j;
    if (vec && j + 4 <= Tk) {
      *reinterpret_cast<f32x4*>(dst) = v4;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < Tk) dst[e] = v4[e];
    }
  };

  auto step = [&](int it, const char* kt) __attribute__((always_inline)) {
    const int j0 = it * kBT;
    const bool edge = (j0 + kBT > kend) || (CAUSAL && j0 + kBT - 1 > qw);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + 32 * hh * ROWB + fr[t]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s, 0, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int jb = j0 + 32 * hh + 16 * m + 8 * g;   // keys jb .. jb+7 in registers 8m .. 8m+7
        f32x4 v4[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * m + e], cs, -l2));
          if (edge) {
            bool ok = jb + e < kend;
            if (CAUSAL) ok = ok && jb + e <= row;
            pe = ok ? pe : 0.f;
          }
          v4[e >> 2][e & 3] = pe;
        }
        // block column chunks 4m + 2g and 4m + 2g + 1 of row c
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          *reinterpret_cast<f32x4*>(st + 32 * c + 4 * ((4 * m + 2 * g + h2) ^ ((c >> 1) & 7))) = v4[h2];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = sr + 8 * i;
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(st + 32 * r + 4 * (sc ^ ((r >> 1) & 7)));
        store4(r, j0 + 32 * hh + 4 * sc, v4);
      }
      __builtin_amdgcn_wave_barrier();
    }
  };

  // tiles past the causal / padding limit of the work-group are zeros, written
  // row-wise (16 lanes cover one row's 64 keys).  Without the causal mask (zero
  // tiles from key padding) one goes out after each computed tile, so the pure
  // writes overlap the computing tiles (+12% on the cross-attention workload);
  // with it the longest-first order already puts the zero-heavy groups last
  const f32x4 z4 = f32x4{};
  int zt = ntiles;
  auto zero_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store4((lane >> 4) + 4 * i, zt * kBT + 4 * (lane & 15), z4);
    ++zt;
  };
  if (ntiles > 0) load_k(0, kb0);
  pipeline_barrier<0>();
  for (int it0 = 0; it0 < ntiles; it0 += 2) {
    static_for<0, 2>([&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      const int it = it0 + u;
      if (it < ntiles) {
        if (it + 1 < ntiles) load_k((it + 1) * kBT, u ? kb0 : kb1);
        if constexpr (kBwdSerialStaging) pipeline_barrier<0>();   // test build only
        step(it, u ? kb1 : kb0);
        if (!CAUSAL && zt < nall) zero_tile();
        pipeline_barrier<0>();
      }
    });
  }
  while (zt < nall) zero_tile();
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <int D, bool C, bool P>
static hipError_t launch_bwd_d(const BwdParams& prm, hipStream_t stream) {
  BwdParams local = prm;
  void* args[] = {&local};
  if (prm.Tq > 0) {
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D, C, P>),
                                         dim3(prm.B * prm.H * prm.n_qtiles), dim3(64 * DqShape<D>::kWaves), args,
                                         0, stream);
    if (e != hipSuccess) return e;
  }
  if (prm.Tk > 0)
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, C, P>),
                           dim3(prm.B * prm.H * prm.n_ktiles), dim3(64 * DkdvShape<D>::kWaves), args, 0, stream);
  return hipSuccess;
}

template <int D>
static hipError_t launch_bwd_mask(const BwdParams& prm, bool causal, bool keypad, hipStream_t stream) {
  if (causal) return keypad ? launch_bwd_d<D, true, true>(prm, stream) : launch_bwd_d<D, true, false>(prm, stream);
  return keypad ? launch_bwd_d<D, false, true>(prm, stream) : launch_bwd_d<D, false, false>(prm, stream);
}

template <int D, bool C, bool P>
static hipError_t launch_weights_d(const WtsParams& prm, hipStream_t stream) {
  WtsParams local = prm;
  void* args[] = {&local};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_weights_kernel<D, C, P>),
                         dim3(prm.B * prm.H * prm.n_qtiles), dim3(kBwdThreads), args, 0, stream);
}

template <int D>
static hipError_t launch_weights_mask(const WtsParams& prm, bool causal, bool keypad, hipStream_t stream) {
  if (causal) return keypad ? launch_weights_d<D, true, true>(prm, stream) : launch_weights_d<D, true, false>(prm, stream);
  return keypad ? launch_weights_d<D, false, true>(prm, stream) : launch_weights_d<D, false, false>(prm, stream);
}

int weights_rows_per_block(int) { return 32 * kBwdWaves; }

hipError_t launch_weights(const WtsParams& prm, int d, bool causal, bool keypad, hipStream_t stream) {
  return d == 64 ? launch_weights_mask<64>(prm, causal, keypad, stream)
                 : launch_weights_mask<128>(prm, causal, keypad, stream);
}

int bwd_rows_per_block(int d) { return d == 128 ? 32 * DqShape<128>::kWaves : 32 * DqShape<64>::kWaves; }
int bwd_keys_per_block(int d) { return d == 128 ? 32 * DkdvShape<128>::kWaves : 32 * DkdvShape<64>::kWaves; }

hipError_t launch_bwd(const BwdParams& prm, int d, bool causal, bool keypad, hipStream_t stream) {
  return d == 64 ? launch_bwd_mask<64>(prm, causal, keypad, stream)
                 : launch_bwd_mask<128>(prm, causal, keypad, stream);
}

}  // namespace attn
