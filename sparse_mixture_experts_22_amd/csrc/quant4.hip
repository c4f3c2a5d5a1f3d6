// 4-bit expert weights: the quantizer and the decode-size expert projections
// that stream them.
//
// The explainer sizes Mixtral at 16 bits and at 4 bits per parameter ("Why
// total and active both matter", Part 4 of "Mixture of Experts: Why Mixtral
// Only Wakes Up Two Specialists") without giving a format; decode batches are
// bound by streaming every touched expert's weights, so 4-bit weights move a
// quarter of the bytes.  Format (per weight stack W[n][R][C], R = reduction):
//   scale s[e][g][c] = bf16_rne(max_{r in group g} |W[e][r][c]| / 7), groups
//   of 128 reduction indices; code q = clamp(rint(W / s), -7, 7) (q = 0 where
//   s = 0), both divisions in fp32; nibble u = q + 8.
//   Codes of expert e: group b = r/128, column tile t = c/16, chunk g =
//   (r%128)/32, column c%16, then 16 bytes = 4 little-endian words; word m
//   holds r = 128b + 32g + 8m + i, element i = 2k in bits 4k..4k+3 and
//   i = 2k+1 in bits 16+4k..16+4k+3 (C a multiple of 16).
// One load instruction of a wave (lane = 16g + c%16) thus reads one
// contiguous kilobyte - a tile's 128 reduction indices - and a wave's four
// tiles are four adjacent kilobytes: streamed in such runs the codes reach
// higher HBM throughput than as separate 128-byte lines per column pair.
// One word ORed into 0x43004300 after masking with 0x000F000F (shifted by
// 4k) gives two bf16 values 128 + u = 136 + q of an MFMA B operand.
//
// Projection kernel (one workgroup of 4 waves per (expert, 128 columns[, K
// split])): lane (c = l%16, g = l/16) of a wave's column tile ct loads the 16
// bytes of the tile's column c, group blk, chunk g: reduction indices 128blk + 32g + 0..31,
// four MFMA B operands (word j: 128blk + 32g + 8j + 0..7).  The A operand of
// lane (row, g) uses the same reduction indices, so each 16x16x32 MFMA j sums
// over 32 indices of one 128-group.  Per group and column tile the MFMAs give
// sum_k x_k (136 + q_k); one extra MFMA chain against a splat of 136 gives
// 136 sum_k x_k (shared by the wave's column tiles), and
//   acc += s[g][col] * (tile - correction)
// applies the scale once per group.  The rest follows the bf16 weight-
// streaming kernels: waves split the reduction, partials are summed in LDS in
// wave order, SwiGLU epilogue (up) or fp32 partial store (down).
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int Q4G = 128;            // reduction indices per scale group
#ifndef MOE_Q4_STAGES
#define MOE_Q4_STAGES 3
#endif
constexpr int Q4_STAGES = MOE_Q4_STAGES;  // blocks of codes in the register ring
constexpr uint32_t kBias136 = 0x4308u;  // bf16 136.0

__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t* __restrict__ W, int n, int R,
                                                          int C, uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ scales) {
  const int G = R / Q4G;
  const int cb = (C + 255) / 256;
  int b = blockIdx.x;
  const int cblk = b % cb;
  b /= cb;
  const int g = b % G;
  const int e = b / G;
  const int c = cblk * 256 + threadIdx.x;
  if (e >= n || c >= C) return;
  const uint16_t* col = W + ((int64_t)e * R + (int64_t)g * Q4G) * C + c;
  float amax = 0.0f;
  for (int r = 0; r < Q4G; ++r) amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)col[(int64_t)r * C] << 16)));
  const uint16_t sbits = f32_to_bf16_rne(amax / 7.0f);
  const float s = __uint_as_float((uint32_t)sbits << 16);
  scales[((int64_t)e * G + g) * C + c] = sbits;
  uint8_t* dst = codes + (int64_t)e * R * (C / 2) + (int64_t)g * C * 64 + (int64_t)(c / 16) * 1024 + (c % 16) * 16;
  for (int jj = 0; jj < 4; ++jj) {  // chunk jj of group g
    u32x4_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t word = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float w = __uint_as_float((uint32_t)col[(int64_t)(32 * jj + 8 * m + i) * C] << 16);
        float q = 0.0f;
        if (s > 0.0f) q = fminf(fmaxf(rintf(w / s), -7.0f), 7.0f);
        const uint32_t u = (uint32_t)((int)q + 8);
        word |= u << (4 * (i >> 1) + 16 * (i & 1));
      }
      out[m] = word;
    }
    *reinterpret_cast<u32x4_t*>(dst + (int64_t)jj * 256) = out;
  }
}

// (x & m) | c in one VALU instruction (the three-operand form takes no
// literal constants and at most one scalar operand, so m is kept in a vector
// register and c in a scalar one; the compiler would otherwise emit a
// separate AND and OR).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "s"(c));
  return r;
}

__device__ __forceinline__ bf16x8_t dq4(uint32_t w, uint32_t m, uint32_t c) {
  u32x4_t r;
  r[0] = and_or(w, m, c);
  r[1] = and_or(w >> 4, m, c);
  r[2] = and_or(w >> 8, m, c);
  r[3] = and_or(w >> 12, m, c);
  return *reinterpret_cast<bf16x8_t*>(&r);
}

// A wave streams TPW 16-column tiles and a workgroup covers 32*TPW columns;
// the launcher picks TPW so that the grid fills whole rounds of resident
// workgroups (two per CU).  Every in-flight load stays in a VGPR.
// MODE 1: up.  Wave w streams matrix w/2 (W1, W3) for column half w%2 over
//         all groups; A rows gathered from x; h = SiLU(a) * b in bf16.
// MODE 2: down.  Wave w streams column half w/2 over half w%2 of this split's
//         groups; o[split] receives the fp32 partial sums.
template <int MODE, int TPW>
__global__ __launch_bounds__(256, 2) void skinny_q4_kernel(
    const uint16_t* __restrict__ A, const int* __restrict__ perm_token,
    const uint8_t* __restrict__ Q1, const uint16_t* __restrict__ S1,
    const uint8_t* __restrict__ Q3, const uint16_t* __restrict__ S3,
    const int* __restrict__ offsets, int n, int Kdim, int N, int splits, int a_rows, int64_t TK,
    uint16_t* __restrict__ hout, float* __restrict__ oout) {
  // ring depth: three blocks while they fit in registers, two for wide waves
  constexpr int STAGES = TPW <= 5 ? Q4_STAGES : 2;
  __shared__ float red[4][4 * TPW][64];

  const int NB = N / (32 * TPW);  // the launcher picks TPW with N % (32*TPW) == 0
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
  const int c16 = lane & 15;
  const int g = lane >> 4;

  constexpr int KPARTS = (MODE == 1) ? 1 : 2;
  const int part = (MODE == 1) ? 0 : (wave & 1);
  const int half = (MODE == 1) ? (wave & 1) : (wave >> 1);
  const int ngr = Kdim / Q4G;
  const int kb0 = (int)((int64_t)sp * ngr / splits);
  const int kb1 = (int)((int64_t)(sp + 1) * ngr / splits);
  const int wb0 = kb0 + (int)((int64_t)part * (kb1 - kb0) / KPARTS);
  const int wb1 = kb0 + (int)((int64_t)(part + 1) * (kb1 - kb0) / KPARTS);

  const bool third = MODE == 1 && wave >= 2;
  const uint8_t* Q = third ? Q3 : Q1;
  const uint16_t* S = third ? S3 : S1;
  // this lane's 16 bytes of column tile 0 in group 0, and its scale column;
  // tile ct adds 1 KiB of codes and 16 scale columns, group blk N*64 bytes.
  // N is a multiple of 32*TPW (chosen by the launcher), so every column exists.
  const int tile0 = nb * 2 * TPW + half * TPW;  // first 16-column tile of this wave
  const int col0 = tile0 * 16 + c16;
  const uint8_t* qsrc = Q + (int64_t)e * Kdim * (N / 2) + (int64_t)tile0 * 1024 + lane * 16;
  const int64_t qtile = 1024;
  const uint16_t* ssrc = S + (int64_t)e * ngr * N + col0;
  // nibble mask and bf16 exponent pattern, uniform (kept in scalar registers)
  uint32_t nib_mask = 0x000F000Fu;
  asm volatile("" : "+v"(nib_mask));  // materialise once in a vector register
  const uint32_t nib_base = __builtin_amdgcn_readfirstlane(0x43004300u);
  bf16x8_t bias;
  {
    const uint32_t bb = kBias136 | (kBias136 << 16);
    u32x4_t t = u32x4_t{bb, bb, bb, bb};
    bias = *reinterpret_cast<bf16x8_t*>(&t);
  }

  for (int m0 = 0; m0 < cnt; m0 += 16) {
    const int rr = (m0 + c16) < cnt ? (m0 + c16) : (cnt - 1);
    const int p = (int)min<int64_t>(max(row_beg + rr, 0), TK - 1);
    const int64_t arow = (MODE == 1) ? (int64_t)min(max(perm_token[p], 0), a_rows - 1) : (int64_t)p;
    const uint16_t* asrc = A + arow * Kdim + g * 32;

    f32x4_t acc[TPW];
#pragma unroll
    for (int ct = 0; ct < TPW; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // register ring of STAGES blocks: the loads of the next STAGES-1
    // blocks are in flight while one block is multiplied
    u32x4_t wq[STAGES][TPW];
    bf16x8_t aq[STAGES][4];
    float sq[STAGES][TPW];
    auto load = [&](int blk, u32x4_t (&w)[TPW], bf16x8_t (&a)[4], float (&s)[TPW]) {
#pragma unroll
      for (int ct = 0; ct < TPW; ++ct) {
        w[ct] = ld_stream(reinterpret_cast<const u32x4_t*>(qsrc + ct * qtile + (int64_t)blk * N * 64));
        s[ct] = __uint_as_float((uint32_t)ssrc[(int64_t)blk * N + ct * 16] << 16);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8_t*>(asrc + (int64_t)blk * Q4G + 8 * j);
    };
    auto block = [&](const u32x4_t (&w)[TPW], const bf16x8_t (&a)[4], const float (&s)[TPW]) {
      f32x4_t corr = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], bias, corr, 0, 0, 0);
#pragma unroll
      for (int ct = 0; ct < TPW; ++ct) {
        f32x4_t t = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], dq4(w[ct][j], nib_mask, nib_base), t, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ct][i] = fmaf(s[ct], t[i] - corr[i], acc[ct][i]);
        // keep one tile's unpacked operands live at a time
        __builtin_amdgcn_sched_barrier(0);
      }
    };
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (wb0 + st < wb1) load(wb0 + st, wq[st], aq[st], sq[st]);
    for (int blk = wb0; blk < wb1; blk += STAGES) {
#pragma unroll
      for (int st = 0; st < STAGES; ++st) {
        const int ahead = blk + st + STAGES - 1;
        if (ahead < wb1)
          load(ahead, wq[(st + STAGES - 1) % STAGES], aq[(st + STAGES - 1) % STAGES],
               sq[(st + STAGES - 1) % STAGES]);
        if (blk + st < wb1) block(wq[st], aq[st], sq[st]);
      }
    }
    // partial tiles -> LDS; slot q = ct*4 + i.  MODE 1: a of column half ch
    // is wave ch's, b is wave 2+ch's; MODE 2: the k halves of column half ch
    // are waves 2ch and 2ch+1.
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < TPW; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][ct * 4 + i][lane] = acc[ct][i];
    __syncthreads();
    {
      const int ch = tid >> 7;           // column half finished by this thread
      const int q0 = ((tid >> 6) & 1) * 2 * TPW;
#pragma unroll
      for (int k = 0; k < 2 * TPW; ++k) {
        const int q = q0 + k;
        const int ct = q >> 2;
        const int i = q & 3;
        const int row = m0 + 4 * (lane >> 4) + i;  // D row of the 16x16 MFMA
        const int colo = (nb * 2 * TPW + ch * TPW + ct) * 16 + (lane & 15);
        if (row >= cnt || colo >= N || row_beg + row >= TK) continue;
        if (MODE == 1) {
          const float va = red[ch][q][lane];
          const float vb = red[2 + ch][q][lane];
          hout[(int64_t)(row_beg + row) * N + colo] = f32_to_bf16_rne(silu_bf16out(va) * vb);
        } else {
          const float v = red[2 * ch][q][lane] + red[2 * ch + 1][q][lane];
          oout[((int64_t)sp * TK + row_beg + row) * N + colo] = v;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize_q4(const uint16_t* W, int n, int R, int C, uint8_t* codes, uint16_t* scales,
                              hipStream_t s) {
  const int G = R / Q4G;
  const int cb = (C + 255) / 256;
  hipLaunchKernelGGL(quantize_q4_kernel, dim3((unsigned)(n * G * cb)), dim3(256), 0, s, W, n, R, C, codes,
                     scales);
  return hipGetLastError();
}

namespace {
// Tiles per wave for a projection with N output columns.  The grid has
// N / (32 * tpw) * mult workgroups, two resident per CU, and a launch takes
// about (rounds of resident workgroups) x (work per workgroup, ~ tpw).  On a
// tie the wider waves win: fewer rounds measured faster (Mixtral decode down
// projection: 512 workgroups of tpw 8 beat 1024 of tpw 4 by 0.7% per layer).
int pick_tpw(int N, int64_t mult, int cus) {
  const int64_t slots = 2 * (int64_t)(cus > 0 ? cus : 256);
  int best = 4;
  int64_t best_cost = -1;
  for (int tpw : {4, 5, 6, 7, 8}) {
    if (N % (32 * tpw) != 0) continue;
    const int64_t wgs = (int64_t)(N / (32 * tpw)) * mult;
    const int64_t cost = (wgs + slots - 1) / slots * tpw;
    if (best_cost < 0 || cost <= best_cost) { best = tpw; best_cost = cost; }
  }
  return best;
}
}  // namespace

hipError_t launch_q4_up(const uint16_t* x, int64_t T, const int* perm_token, const uint8_t* Q1,
                        const uint16_t* S1, const uint8_t* Q3, const uint16_t* S3, const int* offsets,
                        int64_t TK, int n, int d, int f, int cus, uint16_t* h, hipStream_t s) {
  const int tpw = pick_tpw(f, n, cus);
  const dim3 grid((unsigned)(n * (f / (32 * tpw))));
#define MOE_Q4_UP(TPW_)                                                                                   \
  hipLaunchKernelGGL((skinny_q4_kernel<1, TPW_>), grid, dim3(256), 0, s, x, perm_token, Q1, S1, Q3, S3, \
                     offsets, n, d, f, 1, (int)T, TK, h, (float*)nullptr)
  switch (tpw) {
    case 5: MOE_Q4_UP(5); break;
    case 6: MOE_Q4_UP(6); break;
    case 7: MOE_Q4_UP(7); break;
    case 8: MOE_Q4_UP(8); break;
    default: MOE_Q4_UP(4); break;
  }
#undef MOE_Q4_UP
  return hipGetLastError();
}

hipError_t launch_q4_down(const uint16_t* h, const uint8_t* Q2, const uint16_t* S2, const int* offsets,
                          int64_t TK, int n, int f, int d, int splits, int cus, float* o, hipStream_t s) {
  const int tpw = pick_tpw(d, (int64_t)n * splits, cus);
  const dim3 grid((unsigned)(n * (d / (32 * tpw)) * splits));
#define MOE_Q4_DOWN(TPW_)                                                                                  \
  hipLaunchKernelGGL((skinny_q4_kernel<2, TPW_>), grid, dim3(256), 0, s, h, (const int*)nullptr, Q2, S2, \
                     (const uint8_t*)nullptr, (const uint16_t*)nullptr, offsets, n, f, d, splits, (int)TK, TK, \
                     (uint16_t*)nullptr, o)
  switch (tpw) {
    case 5: MOE_Q4_DOWN(5); break;
    case 6: MOE_Q4_DOWN(6); break;
    case 7: MOE_Q4_DOWN(7); break;
    case 8: MOE_Q4_DOWN(8); break;
    default: MOE_Q4_DOWN(4); break;
  }
#undef MOE_Q4_DOWN
  return hipGetLastError();
}

}  // namespace moe
