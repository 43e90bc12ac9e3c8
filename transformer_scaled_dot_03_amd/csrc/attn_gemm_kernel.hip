// Projection GEMM of the multi-head wrapper for gfx950 (MI355X):
//
//   C[M x N] = A[M x K] B[K x N]      bf16 operands and result, fp32 accumulation
//
// A row-major [M x K] (leading dimension lda), B given transposed: Bt = B^T
// row-major [N x K] (ldb), C row-major [M x N] (ldc), leading dimensions in
// elements.  It computes the four projections of multi-head attention -- X W^Q,
// X W^K, X W^V and Concat(heads) W^O ("Attention Is All You Need" notebook
// chapter, section "Multi-Head Self-Attention"; the overview page's MultiHead
// formula).  Shapes there: M = B T rows (any count), K = d_model, N = d_model
// or 3 d_model, multiples of 64 because d_model = h d with d in {64, 128}.
//
// One work-group of 8 waves computes a 256 x 256 tile of C; wave w owns rows
// 64 (w % 4) .. +63 (two 32-row groups) and columns 128 (w / 4) .. +127.  With
// more tiles than CUs the grid is one work-group per CU, each looping over its
// tiles.  The K dimension is walked in steps of 64 through LDS: the A tile
// [256 x 64] and the B^T tile [256 x 64] are copied global -> LDS by
// direct-to-LDS buffer loads, double-buffered (the next step in flight while
// the current one is computed; the next tile's first step in flight during
// this tile's epilogue).  Matrix-core mapping (v_mfma_f32_32x32x16_bf16, lane
// l, g = l / 32, c = l % 32): the product is taken transposed, C^T = B^T A^T --
// the A operand is 16 k of a B^T row, the B operand 16 k of an A row, each one
// 16-byte LDS read (ds_read_b128); the B^T rows of each 32-column block enter
// in an order that leaves every lane of the accumulator with 16 consecutive
// columns of C per block, 64 per row group.  The epilogue rounds to bf16 and
// goes through LDS so that every global store writes whole 256-byte row
// segments (1 KB per instruction).
//
// Rows of A past M and rows of B^T past N read as zero through the buffer
// range check; rows of C past M and columns past N are not written.  A K-step
// of 64 reads 64 KB from L2 per work-group and feeds 256 MFMAs (per wave and
// 16-k slice: 6 KB of fragment reads for 8 MFMAs): measured on MI355X the step
// runs at the matrix-core rate; what remains is the prologue of each tile and
// the burst of output stores that all CUs issue together.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "attn_device.h"
#include "attn_launch.h"

// A test-only build (-DATTN_GEMM_TEST_SERIAL_STAGING=1, built as
// libattn_serial_test.so, never as libattn.so) waits for every direct-to-LDS
// load right after issuing it: no load is in flight while a stage is read, so
// the staging cannot race; its products must equal the pipelined kernel's bit
// for bit.
#ifndef ATTN_GEMM_TEST_SERIAL_STAGING
#define ATTN_GEMM_TEST_SERIAL_STAGING 0
#endif

namespace attn {

namespace {
constexpr int kGemmWaves = 8;
constexpr int kGemmBM = 256;   // rows of C per work-group
constexpr int kGemmBN = 256;   // columns of C per work-group
constexpr int kGemmBK = 64;    // k per pipeline step
}  // namespace

__global__ __launch_bounds__(64 * kGemmWaves, 1) void attn_gemm_bf16_kernel(GemmParams p) {
  constexpr int BK = kGemmBK;
  constexpr int ROWB = BK * 2;                    // 128 B per staged row (A row or B^T row)
  constexpr int STAGE = kGemmBM * ROWB;           // 32 KiB per operand per step
  constexpr int NL = STAGE / 1024 / kGemmWaves;   // 1 KB loads per wave per operand per step
  static_assert(NL == 4 && kGemmBM == kGemmBN, "tile shape");

  // one array per pipeline stage: A rows at +0, B^T rows at +STAGE (a
  // single object per stage lets the compiler see that the epilogue's use of
  // stage 1 never aliases the loads in flight into stage 0)
  __shared__ __attribute__((aligned(1024))) char lds0[2 * STAGE];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * STAGE];
  char* const ab0 = lds0;
  char* const bb0 = lds0 + STAGE;
  char* const ab1 = lds1;
  char* const bb1 = lds1 + STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, c = lane & 31;
  const int wm = w & 3, wn = w >> 2;
  const int nk = p.K / BK;
  const uint32_t lda2 = 2u * p.lda, ldb2 = 2u * p.ldb;

  // ---- tiles of this work-group.  Consecutive work-group ids go to the 8
  // XCDs in turn.  With one tile per work-group the ids are remapped so each
  // XCD gets a contiguous range of tiles; with fewer work-groups than tiles
  // (one per CU, a multiple of 8) the tiles are split into 8 contiguous
  // ranges, one per XCD, dealt round-robin to that XCD's work-groups.  Tile
  // id = row block * column tiles + column tile, so the column tiles of a row
  // block run together on one XCD and share that block of A through its L2.
  const int ntile = p.n_mt * p.n_nt;
  int t_first, t_end, t_step;
  {
    const int pid = blockIdx.x, G = gridDim.x;
    const int xcd = pid % kXcds, idx = pid / kXcds;
    if (G >= ntile) {
      const int per = G / kXcds, rem = G % kXcds;
      t_first = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
      t_end = t_first + 1;
      t_step = 1;
    } else {
      const int per = ntile / kXcds, rem = ntile % kXcds;
      const int start = xcd * per + min(xcd, rem);
      t_first = start + idx;
      t_end = start + per + (xcd < rem ? 1 : 0);
      t_step = G / kXcds;
    }
  }

  // ---- direct-to-LDS staging.  Both operands are stored as 128-byte rows of
  // 8 chunks, chunk q of row R at q ^ k_swz<64>(R).  A: LDS row R = tile row R.
  // B^T: LDS row R = 128 h + 32 i + c holds column 128 h + col(i, c) of the
  // tile, col(i, c) = 64 ((c >> 2) & 1) + 16 i + 4 (c >> 3) + (c & 3): the
  // order that leaves each lane of the accumulator with 16 consecutive columns
  // per 32-column block.
  uint32_t a_src[NL], b_src[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int pos = (kGemmWaves * u + w) * 1024 + 16 * lane;
    const int R = pos / ROWB, pc = (pos % ROWB) / 16;
    a_src[u] = R * lda2 + 16 * (pc ^ k_swz<64>(R));
    const int h = R >> 7, i = (R >> 5) & 3, cc = R & 31;
    const int col = 128 * h + 64 * ((cc >> 2) & 1) + 16 * i + 4 * (cc >> 3) + (cc & 3);
    b_src[u] = col * ldb2 + 16 * (pc ^ k_swz<64>(R));
  }

  struct Tile {
    int m0, n0, arows, brows;
    const __bf16* A;
    const __bf16* B;
  };
  auto tile_at = [&](int t) {
    Tile T;
    const int mt = t / p.n_nt, nt = t - mt * p.n_nt;
    T.m0 = mt * kGemmBM;
    T.n0 = nt * kGemmBN;
    T.arows = min(kGemmBM, p.M - T.m0);
    T.brows = min(kGemmBN, p.N - T.n0);
    T.A = static_cast<const __bf16*>(p.a) + (int64_t)T.m0 * p.lda;
    T.B = static_cast<const __bf16*>(p.bt) + (int64_t)T.n0 * p.ldb;
    return T;
  };
  auto load = [&](const Tile& T, int ks, char* at, char* bt) {
    const int k0 = ks * BK;
    const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(T.A + k0, (uint32_t)(T.arows - 1) * lda2 + ROWB);
    const __amdgpu_buffer_rsrc_t br = buffer_rsrc(T.B + k0, (uint32_t)(T.brows - 1) * ldb2 + ROWB);
#pragma unroll
    for (int u = 0; u < NL; ++u) lds_dma16(ar, at + (kGemmWaves * u + w) * 1024, a_src[u]);
#pragma unroll
    for (int u = 0; u < NL; ++u) lds_dma16(br, bt + (kGemmWaves * u + w) * 1024, b_src[u]);
  };

  // ---- LDS read offsets: lane (c, g), slice t reads chunk 2t + g of row
  // (64 wm + 32 r + c) of A and of row (128 wn + 32 i + c) of B^T
  int rd[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) rd[t] = c * ROWB + 16 * ((2 * t + g) ^ k_swz<64>(c));
  const int a_row0 = 64 * wm * ROWB, b_row0 = 128 * wn * ROWB;

  f32x16 acc[2][4];
  struct Frags {
    bf16x8 a[2];
    bf16x8 b[4];
  };
  auto read_frags = [&](const char* at, const char* bt, int t, Frags& f) {
#pragma unroll
    for (int r = 0; r < 2; ++r) f.a[r] = *reinterpret_cast<const bf16x8*>(at + a_row0 + 32 * r * ROWB + rd[t]);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.b[i] = *reinterpret_cast<const bf16x8*>(bt + b_row0 + 32 * i * ROWB + rd[t]);
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 2; ++r) acc[r][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[i], f.a[r], acc[r][i], 0, 0, 0);
  };
  auto compute = [&](const char* at, const char* bt) {
    Frags f0, f1;
    read_frags(at, bt, 0, f0);
    static_for<0, 4>([&](auto T) {
      constexpr int t = decltype(T)::value;
      Frags& cur = (t % 2 == 0) ? f0 : f1;
      Frags& nxt = (t % 2 == 0) ? f1 : f0;
      if constexpr (t + 1 < 4) read_frags(at, bt, t + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(cur);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- epilogue staging: each wave owns 8 KiB of stage 1 (idle while the
  // next tile's first step loads into stage 0), written as 32 rows x 256 B
  // (chunk q of row r at q ^ (r & 15)) and read back as 4 whole rows per
  // instruction, so every global store writes 1 KB of whole 256-byte row
  // segments.
  char* stg = lds1 + w * 8192;

  Tile cur = tile_at(t_first);
  if (t_first < t_end) load(cur, 0, ab0, bb0);
  for (int t = t_first; t < t_end; t += t_step) {
    pipeline_barrier<0>();
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] = f32x16{};
    int ks = 0;
    for (; ks + 1 < nk; ks += 2) {
      load(cur, ks + 1, ab1, bb1);
      if constexpr (ATTN_GEMM_TEST_SERIAL_STAGING != 0) pipeline_barrier<0>();   // test build only
      compute(ab0, bb0);
      pipeline_barrier<0>();
      if (ks + 2 < nk) load(cur, ks + 2, ab0, bb0);
      if constexpr (ATTN_GEMM_TEST_SERIAL_STAGING != 0) pipeline_barrier<0>();   // test build only
      compute(ab1, bb1);
      pipeline_barrier<0>();
    }
    if (ks < nk) {
      compute(ab0, bb0);
      __builtin_amdgcn_s_barrier();   // every wave is done with buffer 0 before it is refilled
    }
    const Tile done = cur;
    if (t + t_step < t_end) {
      cur = tile_at(t + t_step);
      load(cur, 0, ab0, bb0);
    }
    if constexpr (ATTN_GEMM_TEST_SERIAL_STAGING != 0) pipeline_barrier<0>();   // test build only

    // ---- epilogue: one rounding to bf16, staged through LDS
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 o8;
#pragma unroll
          for (int j = 0; j < 8; ++j) o8[j] = acc[r][i][8 * h2 + j];
          const int q = 8 * g + 2 * i + h2;
          *reinterpret_cast<bf16x8*>(stg + c * 256 + 16 * (q ^ (c & 15))) = __builtin_convertvector(o8, bf16x8);
        }
      const int lc = lane & 15;
      const int col = done.n0 + 128 * wn + 8 * lc;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int rr = 4 * u + (lane >> 4);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stg + rr * 256 + 16 * (lc ^ (rr & 15)));
        const int row = done.m0 + 64 * wm + 32 * r + rr;
        if (row < p.M && col < p.N)
          *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.c) + (int64_t)row * p.ldc + col) = v;
      }
    }
  }
}

// compute units of the device `stream` runs on (the persistent grid size),
// cached per device; the null stream runs on the current device
static int device_cus(hipStream_t stream) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  const hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);   // every thread stores the same value
  }
  return n;
}

hipError_t launch_gemm(const GemmParams& p0, hipStream_t stream) {
  if (p0.M <= 0 || p0.N <= 0) return hipSuccess;
  if (p0.K <= 0 || p0.K % kGemmBK != 0 || p0.N % 8 != 0 || p0.lda % 8 != 0 || p0.ldb % 8 != 0 ||
      p0.ldc % 8 != 0 || p0.lda < p0.K || p0.ldb < p0.K || p0.ldc < p0.N)
    return hipErrorInvalidValue;
  // the buffer ranges are 32-bit: one tile's rows of A and of B^T
  if ((int64_t)kGemmBM * p0.lda * 2 > 0xffffffffLL || (int64_t)kGemmBN * p0.ldb * 2 > 0xffffffffLL)
    return hipErrorInvalidValue;
  GemmParams p = p0;
  p.n_nt = (p.N + kGemmBN - 1) / kGemmBN;
  const int64_t n_mt = (p.M + kGemmBM - 1) / kGemmBM;
  const int64_t ntile = n_mt * p.n_nt;
  if (ntile > 0x7fffffffLL) return hipErrorInvalidValue;
  p.n_mt = static_cast<int>(n_mt);
  // one work-group per tile, or one per CU (a multiple of the 8 XCDs) looping over tiles
  int64_t grid = ntile;
  const int cus = device_cus(stream) / kXcds * kXcds;
  if (cus >= kXcds && ntile > cus) grid = cus;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_gemm_bf16_kernel), dim3(static_cast<unsigned>(grid)),
                         dim3(64 * kGemmWaves), args, 0, stream);
}

// B^T from B: dst [C x R] = src [R x C]^T for up to four matrices (one per
// grid z), 64 x 64 tiles through LDS; R and C multiples of 64
__global__ __launch_bounds__(256) void attn_transpose_kernel(TransposeJobs J) {
  __shared__ __attribute__((aligned(16))) __bf16 tile[64][72];
  const TransposeJob jb = J.job[blockIdx.z];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + 256 * u, r = idx >> 3, ch = idx & 7;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(jb.src + (int64_t)(r0 + r) * J.C + c0 + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[8 * ch + e][r] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + 256 * u, r = idx >> 3, ch = idx & 7;
    *reinterpret_cast<bf16x8*>(jb.dst + (int64_t)(c0 + r) * J.R + r0 + 8 * ch) =
        *reinterpret_cast<const bf16x8*>(&tile[r][8 * ch]);
  }
}

hipError_t launch_transpose(const TransposeJobs& J, int njobs, hipStream_t stream) {
  if (njobs < 1 || njobs > 4 || J.R <= 0 || J.C <= 0 || J.R % 64 != 0 || J.C % 64 != 0) return hipErrorInvalidValue;
  TransposeJobs j = J;
  void* args[] = {&j};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attn_transpose_kernel),
                         dim3(static_cast<unsigned>(J.C / 64), static_cast<unsigned>(J.R / 64), static_cast<unsigned>(njobs)),
                         dim3(256), args, 0, stream);
}

}  // namespace attn
