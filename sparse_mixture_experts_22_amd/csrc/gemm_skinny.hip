// Expert projections for decode-sized batches: few rows per expert, so the
// cost is streaming every touched expert's weights from HBM once.
//
// The pages note that a sparse MoE holds all experts' parameters in memory
// while a token uses only its two ("Why total and active both matter", Part 4
// of "Mixture of Experts: Why Mixtral Only Wakes Up Two Specialists"); with a
// small batch every expert is still touched, and the layer is bound by reading
// 3*d*f bf16 weights per touched expert.
//
// Work unit: one workgroup per (expert, column block[, K split]); each wave
// streams a 128-column chunk of one matrix.  The up projection's workgroup has
// 8 waves over 512 columns of W1 and the same 512 of W3, so it reads 1 KiB
// contiguous bytes of each weight row it touches; the down projection's has 4
// waves over 256 columns of W2, two per K half.  Longer row segments and fewer
// concurrent streams read faster (probes: 1 KiB segments 6.3-6.5 TB/s, 512 B
// 6.0-6.3, 256 B 5.7); the 1 KiB up blocks took the Mixtral decode up
// projection from 313 to 301 us, while 512-column down blocks (four K splits
// to fill the chip) measured slower than these.  A decode launch is resident
// in one round.  Each lane loads 8 rows x 16 bytes of the weight block (one 8x8 bf16
// block), transposes it in registers and feeds eight v_mfma_f32_16x16x32_bf16
// directly as B operands - the weights never pass through LDS.  The MFMA column index c of fragment j stands for
// weight column col0 + c*8 + j.  A fragments (16 token rows) come straight
// from global memory (x or h is tiny and stays in L2).  Loads of the next K
// step are issued before the MFMAs of the current one.  The waves' partial tiles
// are summed in LDS in wave order (fixed order, deterministic), then the
// SwiGLU epilogue (up) or the fp32 store of a partial sum (down) follows.
// Rows beyond 16 per expert are handled by further passes over the weights.
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ void transpose8x8(const u32x4_t (&in)[8], bf16x8_t (&out)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t r0 = in[2 * q][p];
      const uint32_t r1 = in[2 * q + 1][p];
      lo[q] = __builtin_amdgcn_perm(r1, r0, 0x05040100u);
      hi[q] = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
    }
    u32x4_t l = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
    u32x4_t h = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
    out[2 * p] = *reinterpret_cast<bf16x8_t*>(&l);
    out[2 * p + 1] = *reinterpret_cast<bf16x8_t*>(&h);
  }
}

// Lanes whose columns lie past N read column 0's rows instead (the caller
// clamps src), so every load is in bounds; those columns are never stored.
__device__ __forceinline__ void load_block(u32x4_t (&q)[8], const uint16_t* src, int64_t row_stride) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
    q[r] = ld_stream(reinterpret_cast<const u32x4_t*>(src + (int64_t)r * row_stride));
}

__device__ __forceinline__ void mma_block(const u32x4_t (&q)[8], const bf16x8_t& a, f32x4_t (&acc)[8]) {
  bf16x8_t fr[8];
  transpose8x8(q, fr);
#pragma unroll
  for (int c = 0; c < 8; ++c)
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, fr[c], acc[c], 0, 0, 0);
}

// MODE 1: up.  Wave w streams matrix w/4 (W1, W3) over the whole of K for
//         column chunk w%4; A rows are gathered from x via perm_token;
//         h = SiLU(a) * b in bf16.
// MODE 2: down.  Wave w streams W2 for column chunk w/2 over half w%2 of this
//         split's K range; A rows are h; o[split] receives the fp32 partial sum.
// With the ping-pong buffers a wave keeps two K steps of loads in flight
// (8 waves per CU).  The variant without them fits 4 workgroups per CU
// (a decode launch is resident in one round) but measured slower: per-wave
// memory parallelism matters more here than occupancy.
#ifndef MOE_SKINNY_PINGPONG
#define MOE_SKINNY_PINGPONG 1
#endif
constexpr int SKINNY_OCC = MOE_SKINNY_PINGPONG ? 2 : 4;

// Waves per workgroup and weight columns per workgroup: the up projection
// runs 8 waves (4 column quarters of W1 and the same 4 of W3), so a workgroup
// reads 1 KiB of each of its two matrices' rows; the down projection runs 4.
template <int MODE> struct SkinnyShape {
  static constexpr int kWaves = MODE == 1 ? 8 : 4;
  static constexpr int kCols = MODE == 1 ? 512 : 256;
};

template <int MODE>
__global__ __launch_bounds__(SkinnyShape<MODE>::kWaves * 64, SKINNY_OCC * 4 / SkinnyShape<MODE>::kWaves) void skinny_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int* __restrict__ offsets, int n, int Kdim, int N, int splits, int a_rows, int64_t TK,
    uint16_t* __restrict__ hout, float* __restrict__ oout) {
  constexpr int NW = SkinnyShape<MODE>::kWaves;
  constexpr int NCOL = SkinnyShape<MODE>::kCols;
  constexpr int NCH = NCOL / 128;  // 128-column chunks per workgroup
  __shared__ float red[NW][32][64];  // per-wave partial accumulators

  const int NB = (N + NCOL - 1) / NCOL;
  int bid = blockIdx.x;
  const int sp = bid % splits;
  bid /= splits;
  const int nb = bid % NB;
  const int e = bid / NB;
  if (e >= n) return;
  const int row_beg = offsets[e];
  const int cnt = offsets[e + 1] - row_beg;
  if (cnt <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  // reduction range and column chunk of this wave, in steps of 32
  constexpr int KPARTS = (MODE == 1) ? 1 : 2;
  const int part = (MODE == 1) ? 0 : (wave & 1);
  const int half = (MODE == 1) ? (wave % NCH) : (wave >> 1);
  const int nkc = Kdim / 32;
  const int kc0 = (int)((int64_t)sp * nkc / splits);
  const int kc1 = (int)((int64_t)(sp + 1) * nkc / splits);
  const int wk0 = kc0 + (int)((int64_t)part * (kc1 - kc0) / KPARTS);
  const int wk1 = kc0 + (int)((int64_t)(part + 1) * (kc1 - kc0) / KPARTS);

  const int col0 = nb * NCOL + half * 128 + r16 * 8;
  const bool b_ok = col0 < N;
  const uint16_t* bmat = (MODE == 1 && wave >= NCH) ? B3 : B1;
  const uint16_t* bsrc = bmat + (int64_t)e * Kdim * N + (b_ok ? col0 : 0) + (int64_t)(g * 8) * N;
  const int64_t kstep = (int64_t)32 * N;

  for (int m0 = 0; m0 < cnt; m0 += 16) {
    const int rr = (m0 + r16) < cnt ? (m0 + r16) : (cnt - 1);
    const int p = (int)min<int64_t>(max(row_beg + rr, 0), TK - 1);
    const int64_t arow = (MODE == 1) ? (int64_t)min(max(perm_token[p], 0), a_rows - 1) : (int64_t)p;
    const uint16_t* asrc = A + arow * Kdim + g * 8;

    f32x4_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#if MOE_SKINNY_PINGPONG
    // ping-pong: step kc in (qa, aa), step kc+1 in (qb, ab).  The loads are
    // unconditional (indices clamped to the last step) and scheduling
    // barriers fence each phase, so the compiler waits only for the buffer
    // about to be multiplied; a conditional load here makes it wait for all.
    u32x4_t qa[8], qb[8];
    bf16x8_t aa, ab;
    int kc = wk0;
    if (kc < wk1) {
      load_block(qa, bsrc + kc * kstep, N);
      aa = *reinterpret_cast<const bf16x8_t*>(asrc + kc * 32);
    }
    while (kc < wk1) {
      {
        const int k1 = min(kc + 1, wk1 - 1);
        load_block(qb, bsrc + k1 * kstep, N);
        ab = *reinterpret_cast<const bf16x8_t*>(asrc + k1 * 32);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma_block(qa, aa, acc);
      __builtin_amdgcn_sched_barrier(0);
      {
        const int k2 = min(kc + 2, wk1 - 1);
        load_block(qa, bsrc + k2 * kstep, N);
        aa = *reinterpret_cast<const bf16x8_t*>(asrc + k2 * 32);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kc + 1 >= wk1) ab = bf16x8_t{};  // past the end: a zero A fragment adds nothing
      mma_block(qb, ab, acc);
      __builtin_amdgcn_sched_barrier(0);
      kc += 2;
    }
#else
    for (int kc = wk0; kc < wk1; ++kc) {
      u32x4_t q[8];
      load_block(q, bsrc + kc * kstep, N);
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(asrc + kc * 32);
      mma_block(q, a, acc);
    }
#endif
    // partial tiles -> LDS; register slot q = c*4 + j
    __syncthreads();  // previous pass finished reading red
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][c * 4 + j][lane] = acc[c][j];
    __syncthreads();
    // thread (qg = tid/64, lane) finishes slots q = qg*QPT .. qg*QPT+QPT-1 of
    // every 128-column chunk.  MODE 1: a of chunk ch is wave ch's, b is wave
    // NCH+ch's; MODE 2: the two k halves of chunk ch are waves 2ch and 2ch+1.
    constexpr int QPT = 32 / NW;
    const int qg = tid >> 6;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const int q = qg * QPT + i;
        const int c = q >> 2;
        const int j = q & 3;
        const int row = m0 + 4 * (lane >> 4) + j;  // D row of the 16x16 MFMA
        const int colo = nb * NCOL + ch * 128 + (lane & 15) * 8 + c;
        if (row >= cnt || colo >= N || row_beg + row >= TK) continue;
        if (MODE == 1) {
          const float va = red[ch][q][lane];
          const float vb = red[NCH + ch][q][lane];
          hout[(int64_t)(row_beg + row) * N + colo] = f32_to_bf16_rne(silu_bf16out(va) * vb);
        } else {
          const float v = red[2 * ch][q][lane] + red[2 * ch + 1][q][lane];
          oout[((int64_t)sp * TK + row_beg + row) * N + colo] = v;
        }
      }
  }
}

}  // namespace

hipError_t launch_skinny_up(const uint16_t* x, int64_t T, const int* perm_token, const uint16_t* W1,
                            const uint16_t* W3, const int* offsets, int64_t TK, int n, int d, int f,
                            uint16_t* h, hipStream_t s) {
  constexpr int NCOL = SkinnyShape<1>::kCols;
  const int NB = (f + NCOL - 1) / NCOL;
  hipLaunchKernelGGL((skinny_kernel<1>), dim3((unsigned)(n * NB)), dim3(SkinnyShape<1>::kWaves * 64), 0, s, x, perm_token,
                     W1, W3, offsets, n, d, f, 1, (int)T, TK, h, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_skinny_down(const uint16_t* h, const uint16_t* W2, const int* offsets, int64_t TK,
                              int n, int f, int d, int splits, float* o, hipStream_t s) {
  constexpr int NCOL = SkinnyShape<2>::kCols;
  const int NB = (d + NCOL - 1) / NCOL;
  hipLaunchKernelGGL((skinny_kernel<2>), dim3((unsigned)(n * NB * splits)), dim3(SkinnyShape<2>::kWaves * 64), 0, s, h,
                     (const int*)nullptr, W2, (const uint16_t*)nullptr, offsets, n, f, d, splits,
                     (int)TK, TK, (uint16_t*)nullptr, o);
  return hipGetLastError();
}

}  // namespace moe
