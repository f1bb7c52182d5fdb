// Small-M (decode) FP8 block-scaled NT GEMM for gfx950.
//
// Same operation as the tiled kernel (FP8 block-quantised GEMM page on
// lpnh.cn, s2.2 and s3.2; NT layout per the DeepGEMM page on pzsr.cn, s3.1),
// for M <= 64 where the work is bound by streaming B (N x K bytes) from HBM:
// the lpnh.cn page (s3.4, s4.3, s5.5) notes that the kernel picks its tile and
// pipeline depth from the shape, and that on small problems loading the
// scales/operands rather than arithmetic dominates.
//
// gfx950 mapping
//  * A workgroup (4 waves) owns 128 (or 64) rows of B inside one 128-row scale
//    block and a contiguous range of K blocks.  B streams through a 3-stage
//    LDS ring fed by global_load_lds_dwordx4 (16 KB of B per stage, 8 consecutive lanes per
//    128-byte row, chunk permutation as in the tiled kernel); a workgroup
//    needs <= 75 KB of LDS, so two run per CU with 4 stages (64 KB) of B in
//    flight between them.  A (M padded to 16/32/64 rows, rows past M clamped)
//    and its 1x128 (or 128x128) scales, and the B block scale, ride in the
//    same stages.  The ring slots are distinct __shared__ arrays and the loop
//    is unrolled by the ring depth, so the compiler's LDS-DMA dependency
//    tracking can see that the slot being filled is not the slot being read
//    (with one array it waits for every outstanding load before each read).
//  * Each wave computes 32 (or 16) rows of B x MP columns of A with
//    v_mfma_f32_16x16x128_f8f6f4 (B rows drive the instruction's first
//    operand), promoting each 128-K partial with sa*sb in FP32.
//  * Split-K when N/128 workgroups cannot fill the GPU: split s writes its
//    FP32 partial tile to the caller's workspace, then the last split to
//    arrive (device-scope counter) sums the S partials in split order and
//    writes BF16, so the result does not depend on arrival order.  The
//    arrival counters sit in the first kSplitkCounterBytes of the same
//    workspace (one int per tile, a fixed region whatever the shape); the
//    caller hands the workspace over zeroed once, and the reducing workgroup
//    resets its counter, so every call leaves the region zeroed again.  The
//    library keeps no state of its own: calls with distinct workspaces may
//    overlap on one GPU.
#include "dg_device.hpp"
#include "dg_internal.hpp"

#include <stdlib.h>

namespace dg {
namespace {

constexpr int BN = 128;
constexpr int BK = 128;
constexpr int kMaxNS = 8;          // deepest LDS ring (named slot arrays l0 .. l7)
constexpr int kMaxCounters = (int)(kSplitkCounterBytes / 4);  // tiles: N up to 1M with 128-row tiles
constexpr int kMaxSplits = 16;

// Form of the A operand: E4M3 codes with their scales, or FP32 / BF16 values
// the kernel quantises itself with 1x128 blocks.
enum AForm { A_CODES = 0, A_F32 = 1, A_BF16 = 2 };

struct SkinnyArgs {
  uint16_t* c;
  Epilogue epi;
  const uint8_t* a;
  const void* af;   // FP32 or BF16 A when the kernel quantises A itself, else null
  const uint32_t* sfa;  // E8: packed UE8M0 exponents (four K blocks per word)
  const uint32_t* sfb;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  float* partials;  // split s at partials + s * part_stride, row-major [.][N], when S > 1
  int* counters;    // per-tile arrival counters (zero on entry, left zero), when S > 1
  int64_t part_stride;
  int a_block_rows;
  int M, N, K;
  int nkb;
  int sa_stride;  // ceil(M / a_block_rows)  (masked: ceil(max_m / a_block_rows))
  int sb_stride;  // ceil(N / 128)
  int S;          // K splits
  // masked grouped layout: group g has max_m rows of A and C, masked_m[g] of
  // them valid; the grid covers groups x chunks (MP rows each) x N tiles
  const int32_t* masked_m;
  int max_m, chunks, tiles;
};

__device__ __forceinline__ int lds_swz(int r) { return ((r & 3) << 1) ^ ((r >> 2) & 1); }

__device__ __forceinline__ v8i read_frag(const uint8_t* lds, int row_base, int off0, int off1) {
  const v4i lo = *reinterpret_cast<const v4i*>(lds + row_base * 128 + off0);
  const v4i hi = *reinterpret_cast<const v4i*>(lds + row_base * 128 + off1);
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// The end of a small-M tile: lane (wave, l) holds acc[f][i] = C[m = 16i + l%16][n = n0 +
// 16*F*wave + 16f + 4*(l/16) + r], r = 0..3.  Without split-K it stores BF16
// (with the epilogue); with split-K it publishes its FP32 partial tile, and
// the last split to arrive sums all S partials in split order and stores.
template <int MP, int F>
__device__ __forceinline__ void skinny_finish(const SkinnyArgs& p, const v4f (&acc)[F][MP / 16],
                                              int tile, int split, int n0, int lane, int wave,
                                              int& s_last) {
  constexpr int NI = MP / 16;
  constexpr int BNT = 64 * F;
  const int fr = lane & 15;
  if (p.S == 1) {
    with_epilogue(p.epi, [&](auto act, auto res) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int m = 16 * i + fr;
        if (m >= p.M) continue;
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const int n = n0 + wave * 16 * F + 16 * f + 4 * (lane >> 4);
          if (n < p.N) {
            const float t[4] = {acc[f][i][0], acc[f][i][1], acc[f][i][2], acc[f][i][3]};
            store4<decltype(act)::value, decltype(res)::value != 0>(p.c, m, n, t, p.epi);
          }
        }
      }
    });
    return;
  }

  // split-K.  The 8 XCDs have separate L2s, so the partials are published
  // with device-scope (relaxed atomic) stores, which are written through to
  // the device-coherent level, and read back with device-scope loads; a full
  // __threadfence() would instead write back each XCD's whole L2.
  float* mine = p.partials + (int64_t)split * p.part_stride;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int m = 16 * i + fr;
    if (m >= p.M) continue;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int n = n0 + wave * 16 * F + 16 * f + 4 * (lane >> 4);
      if (n < p.N) {
        uint64_t* d = reinterpret_cast<uint64_t*>(mine + (int64_t)m * p.N + n);
        const uint64_t lo = (uint64_t)__float_as_uint(acc[f][i][0]) |
                            ((uint64_t)__float_as_uint(acc[f][i][1]) << 32);
        const uint64_t hi = (uint64_t)__float_as_uint(acc[f][i][2]) |
                            ((uint64_t)__float_as_uint(acc[f][i][3]) << 32);
        __hip_atomic_store(d, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // every store of this wave has completed (is device-visible) ...
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  __syncthreads();  // ... and so have those of every wave of the workgroup
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(&p.counters[tile], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == p.S - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // The last split sums the S partials in split order (deterministic) and
  // writes BF16.  Thread t owns the float4 positions t + 256 j of the
  // M x 128 tile; the loads of G splits x PJ positions are issued together so
  // that one memory latency covers them, then added in split order.
  constexpr int PJ = MP * (BNT / 4) / 256;         // positions per thread: 1 .. 8
  constexpr int G = 16 / PJ;                        // splits loaded per round
  const int ncols = min(BNT, p.N - n0);
  float4 sum[PJ];
  bool live[PJ];
  int64_t off[PJ];
  int pm[PJ], pn[PJ];
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int idx = threadIdx.x + 256 * j;
    const int m = idx / (BNT / 4);
    const int cc = (idx - m * (BNT / 4)) * 4;
    live[j] = m < p.M && cc < ncols;
    off[j] = (int64_t)m * p.N + n0 + cc;
    pm[j] = m;
    pn[j] = n0 + cc;
    sum[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int s0 = 0; s0 < p.S; s0 += G) {
    uint64_t part[G][PJ][2];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        const int sp = s0 + g;
        if (sp < p.S && live[j]) {
          const uint64_t* src =
              reinterpret_cast<const uint64_t*>(p.partials + (int64_t)sp * p.part_stride + off[j]);
          part[g][j][0] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          part[g][j][1] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        if (s0 + g < p.S && live[j]) {
          const float4 v = make_float4(__uint_as_float((uint32_t)part[g][j][0]),
                                       __uint_as_float((uint32_t)(part[g][j][0] >> 32)),
                                       __uint_as_float((uint32_t)part[g][j][1]),
                                       __uint_as_float((uint32_t)(part[g][j][1] >> 32)));
          if (s0 + g == 0) {
            sum[j] = v;
          } else {
            sum[j].x += v.x; sum[j].y += v.y; sum[j].z += v.z; sum[j].w += v.w;
          }
        }
      }
  }
  with_epilogue(p.epi, [&](auto act, auto res) {
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      if (!live[j]) continue;
      const float t[4] = {sum[j].x, sum[j].y, sum[j].z, sum[j].w};
      store4<decltype(act)::value, decltype(res)::value != 0>(p.c, pm[j], pn[j], t, p.epi);
    }
  });
  if (threadIdx.x == 0)  // leave the counter zeroed for the next call
    __hip_atomic_store(&p.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// AF = A_F32 / A_BF16: A arrives as FP32 or BF16 values and the workgroup
// quantises it with 1x128 blocks: each stage also carries the A block (MP
// rows x 128 values, rows past M clamped), fetched by the same LDS DMA as B.
// After the step's barrier, the TPR = 256 / MP consecutive threads of row
// t / TPR read its 16-byte chunks j, j + TPR, j + 2 TPR, ... (j = t % TPR),
// share the row's amax through lane exchanges and encode their values; the
// codes (in the layout the A DMA produces) and the row scales go to a code
// buffer, and a second barrier publishes them to the MFMAs.  BF16 values are
// widened to FP32 exactly, so the codes and scales are those of the FP32
// quantiser on the widened values.  A is staged through LDS rather than
// registers: the compiler waits for every load in flight before using a
// register loaded ahead of LDS DMA instructions, which would drain the ring
// each step.
// E8: power-of-two (UE8M0) scales (DeepGEMM page on pzsr.cn, s3.1): the
// stages carry the packed exponent words in place of the FP32 scales, the
// scaled MFMA applies them and the accumulators chain through K.
// NS: LDS ring depth; NS - 1 stages are in flight while one is consumed.
// Measured on MI355X over the nine decode shapes: 4 or 6 slots (one
// workgroup per CU) are no faster than 3 at the best split count, so the
// launches use 3.
// MASKED: the masked grouped layout (a reading of the grouped GEMM of the
// pzsr.cn DeepGEMM page, s2.3 and s3.2, for decode-time MoE): workgroup
// (g, chunk, N tile, split) computes rows [chunk * MP, chunk * MP + MP) of
// group g that are below masked_m[g] (clamped into [0, max_m]), with A, the
// scales, B and C offset to that group; a chunk with no valid row exits.
template <int MP, int F, int AF = A_CODES, bool E8 = false, int NS = 3, bool MASKED = false>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(SkinnyArgs args) {
  constexpr bool AQ = AF != A_CODES;              // A quantised in the kernel
  static_assert(!(AQ && E8), "in-kernel quantisation uses FP32 scales");
  static_assert(!(MASKED && AQ), "masked layout: E4M3 A");
  constexpr int ESZ = AF == A_F32 ? 4 : 2;        // bytes per staged A value (AQ)
  constexpr int ARB = BK * ESZ;                   // bytes per staged A row (AQ)
  constexpr int TPR = 256 / MP;                   // quantising threads per A row (AQ)
  constexpr int CPT = ARB / 16 / TPR;             // 16-byte chunks per thread (AQ)
  constexpr int BNT = 64 * F;                     // B rows per workgroup (F fragments per wave)
  constexpr int MPE = MP < 32 ? 32 : MP;          // A rows staged (>= 4 DMA instructions)
  constexpr int B_BYTES = BNT * BK;               // 8 or 16 KB
  constexpr int A_BYTES = AQ ? MP * ARB : MPE * BK;  // FP32 / BF16 A, or E4M3 A
  constexpr int SA_BYTES = AQ ? 0 : 4 * 256;      // one 64-float copy per wave
  constexpr int SB_BYTES = 4 * 256;               // B block scale (64 copies) per wave
  constexpr int STAGE = B_BYTES + A_BYTES + SA_BYTES + SB_BYTES;
  constexpr int B_IT = B_BYTES / 1024 / 4;        // DMA instructions per wave per stage
  constexpr int A_IT = A_BYTES / 1024 / 4;
  constexpr int PER_STAGE = B_IT + A_IT + (AQ ? 1 : 2);  // + the A scale row + the B scale
  constexpr int NI = MP / 16;                     // A fragments
  constexpr int QB_BYTES = AQ ? MP * BK + MP * 4 : 16;  // code buffer: codes, then row scales
  static_assert(!AQ || (A_IT >= 1 && CPT >= 1 && (ARB / 16) % TPR == 0 && (CPT & (CPT - 1)) == 0),
                "A staging");
  static_assert(NS >= 3 && NS <= kMaxNS, "ring depth");
  static_assert((NS - 2) * PER_STAGE <= 63, "s_waitcnt vmcnt range");
  static_assert(NS * STAGE + (AQ ? QB_BYTES : 0) <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t l0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t l1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t l2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t l3[NS > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t l4[NS > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t l5[NS > 5 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t l6[NS > 6 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t l7[NS > 7 ? STAGE : 16];
  // AQ code buffer: MP rows x 128 codes, then the MP row scales (never a DMA
  // target, so stores to it need no wait on the DMA in flight)
  __shared__ __attribute__((aligned(128))) uint8_t qb[QB_BYTES];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile = blockIdx.x / args.S;  // also the split-K counter index
  const int split = blockIdx.x - tile * args.S;
  SkinnyArgs p = args;
  int nt = tile;
  if constexpr (MASKED) {
    const int gc = tile / p.tiles;
    nt = tile - gc * p.tiles;
    const int g = gc / p.chunks;
    const int r0 = (gc - g * p.chunks) * MP;
    int valid = p.masked_m[g];
    valid = valid < 0 ? 0 : (valid > p.max_m ? p.max_m : valid);
    const int rows = valid - r0 < MP ? valid - r0 : MP;
    if (rows <= 0) return;  // uniform: before any barrier
    const int64_t row0 = (int64_t)g * p.max_m + r0;
    p.a += row0 * p.K;
    p.b += (int64_t)g * p.N * p.K;
    if constexpr (E8) {  // UE8M0 words: four K blocks each, per-group arrays
      const int64_t nw = (p.nkb + 3) / 4;
      p.sfa += g * nw * p.sa_stride + (p.a_block_rows == 1 ? r0 : r0 / 128);
      p.sfb += g * nw * p.sb_stride;
    } else {
      p.sa += (int64_t)g * p.nkb * p.sa_stride + (p.a_block_rows == 1 ? r0 : r0 / 128);
      p.sb += (int64_t)g * p.nkb * p.sb_stride;
    }
    p.c += row0 * p.epi.ldc;  // (N / 2 columns with SwiGLU)
    if (p.epi.res) p.epi.res += row0 * p.epi.ldc;
    if (p.S > 1) p.partials += row0 * p.N;
    p.M = rows;
  }
  const int n0 = nt * BNT;
  const int kb0 = (int)((int64_t)split * p.nkb / p.S);
  const int kb1 = (int)((int64_t)(split + 1) * p.nkb / p.S);
  const int nk = kb1 - kb0;  // >= 1 (S <= nkb)

  // DMA source offsets (bytes, at kb = 0).  Instruction j of wave w fills the
  // 1 KB at LDS offset (j*4 + w)*1024 of the B (or A) region: rows 8*(j*4+w)
  // .. +7, lane L -> row +L/8, physical chunk L%8.
  uint32_t boff[B_IT], aoff[A_IT];
  const uint8_t* a32[AQ ? A_IT : 1];  // AQ: instruction j's A row chunk at kb = 0
#pragma unroll
  for (int j = 0; j < B_IT; ++j) {
    const int r = (j * 4 + wave) * 8 + (lane >> 3);
    int gr = n0 + r;
    gr = gr < p.N ? gr : p.N - 1;
    boff[j] = (uint32_t)gr * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ lds_swz(r)) * 16);
  }
#pragma unroll
  for (int j = 0; j < A_IT; ++j) {
    if constexpr (AQ) {
      // 1 KB = 1024 / ARB rows: lane L -> row + L / LPR, bytes 16 (L % LPR)
      constexpr int LPR = ARB / 16;
      const int r = (j * 4 + wave) * (64 / LPR) + lane / LPR;
      const int gr = r < p.M ? r : p.M - 1;
      a32[j] = static_cast<const uint8_t*>(p.af) + ((int64_t)gr * p.K * ESZ + (lane % LPR) * 16);
      aoff[j] = 0;
    } else {
      const int r = (j * 4 + wave) * 8 + (lane >> 3);
      const int gr = r < p.M ? r : p.M - 1;
      aoff[j] = (uint32_t)gr * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ lds_swz(r)) * 16);
    }
  }
  const int sa_row = p.a_block_rows == 1 ? (lane < p.M ? lane : p.M - 1) : 0;
  const int nb = n0 / 128;  // the 128 rows of this workgroup form one B scale block

  auto issue_stage = [&](int it, uint8_t* st) {
    const int kb = kb0 + (it < nk ? it : nk - 1);  // past the range: re-stage the last block
#pragma unroll
    for (int j = 0; j < B_IT; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(p.b + boff[j] + (uint32_t)kb * BK),
                                       (__attribute__((address_space(3))) void*)(st + (j * 4 + wave) * 1024),
                                       16, 0, 0);
    if constexpr (AQ) {
#pragma unroll
      for (int j = 0; j < A_IT; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(a32[j] + (int64_t)kb * ARB),
                                         (__attribute__((address_space(3))) void*)(st + B_BYTES + (j * 4 + wave) * 1024),
                                         16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < A_IT; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(p.a + aoff[j] + (uint32_t)kb * BK),
                                         (__attribute__((address_space(3))) void*)(st + B_BYTES + (j * 4 + wave) * 1024),
                                         16, 0, 0);
      const void* sa_src = E8 ? (const void*)(p.sfa + (int64_t)(kb >> 2) * p.sa_stride + sa_row)
                              : (const void*)(p.sa + (int64_t)kb * p.sa_stride + sa_row);
      __builtin_amdgcn_global_load_lds(sa_src,
                                       (__attribute__((address_space(3))) void*)(st + B_BYTES + A_BYTES + wave * 256),
                                       4, 0, 0);
    }
    const void* sb_src = E8 ? (const void*)(p.sfb + (int64_t)(kb >> 2) * p.sb_stride + nb)
                            : (const void*)(p.sb + (int64_t)kb * p.sb_stride + nb);
    __builtin_amdgcn_global_load_lds(sb_src,
                                     (__attribute__((address_space(3))) void*)(st + B_BYTES + A_BYTES + SA_BYTES + wave * 256),
                                     4, 0, 0);
  };

  // in-kernel quantisation of A (AQ): row qr, 16-byte chunks
  // qj + TPR ((i + qr) mod CPT): the TPR threads of a row read consecutive
  // chunks, and each row starts its rotation at a different group of TPR
  // chunks, so the rows a wave reads together fall on different LDS banks
  // (without the rotation the 512-byte FP32 rows of a 64-row block all start
  // on the same bank: half of the LDS cycles were bank conflicts)
  const int qr = threadIdx.x / TPR;
  const int qj = threadIdx.x % TPR;
  int qc[CPT];  // chunk read by step i
#pragma unroll
  for (int i = 0; i < CPT; ++i) qc[i] = qj + TPR * ((i + qr) & (CPT - 1));
  auto quantise_a = [&](const uint8_t* st) {
    // read as integers: a float-typed LDS read makes the compiler wait for
    // every DMA in flight (it cannot tell it from the ring's other slots)
    v4i raw[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      raw[i] = *reinterpret_cast<const v4i*>(st + B_BYTES + qr * ARB + 16 * qc[i]);
    constexpr int NV = CPT * 16 / ESZ / 4;  // float4 groups per thread
    float4 v[NV];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if constexpr (AF == A_F32) {
        v[i] = make_float4(__int_as_float(raw[i][0]), __int_as_float(raw[i][1]),
                           __int_as_float(raw[i][2]), __int_as_float(raw[i][3]));
      } else {  // BF16 -> FP32 is exact: the bits move to the top half
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w0 = (uint32_t)raw[i][2 * h], w1 = (uint32_t)raw[i][2 * h + 1];
          v[2 * i + h] = make_float4(__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                                     __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u));
        }
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) m = abs_max4(m, v[i]);
    const BlockScale bs = block_scale(lane_group_max<TPR>(m));
    // code byte k of row qr sits in logical 16-byte chunk k / 16, at physical
    // chunk (k / 16) ^ swz(qr); float4 group g of this thread holds values
    // [4 G, 4 G + 4) of the row with G = its global group index
    const int sw = lds_swz(qr);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = qc[i / (16 / ESZ / 4)];  // source chunk of group i
      const int g = c * (16 / ESZ / 4) + i % (16 / ESZ / 4);
      const int k = 4 * g;
      *reinterpret_cast<uint32_t*>(qb + qr * 128 + ((((k >> 4) ^ sw) << 4) | (k & 15))) =
          encode4_block(v[i], bs);
    }
    if (qj == 0) reinterpret_cast<float*>(qb + MP * BK)[qr] = bs.s;
  };

  const int fr = lane & 15;
  const int off0 = fr * 128 + (((2 * (lane >> 4)) ^ lds_swz(fr)) * 16);
  const int off1 = fr * 128 + (((2 * (lane >> 4) + 1) ^ lds_swz(fr)) * 16);

  v4f acc[F][NI];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[f][i] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  // ring slot i (one named array per slot: see above)
  auto slot = [&](auto tag) -> uint8_t* {
    constexpr int i = decltype(tag)::value;
    if constexpr (i == 0) return l0;
    else if constexpr (i == 1) return l1;
    else if constexpr (i == 2) return l2;
    else if constexpr (i == 3) return l3;
    else if constexpr (i == 4) return l4;
    else if constexpr (i == 5) return l5;
    else if constexpr (i == 6) return l6;
    else return l7;
  };
  // stages 0 .. NS-2 go into slots 0 .. NS-2; stage s always lives in slot s % NS
  static_for<NS - 1>([&](auto tag) { issue_stage(decltype(tag)::value, slot(tag)); });

  // one K block: stage `it` sits in `cur`; stage it+NS-1 goes into `nxt`
  // (the slot of stage it-1, free once every wave has passed this barrier)
  auto body = [&](int it, const uint8_t* cur, uint8_t* nxt) {
    // this wave's loads for stage `it` have landed once at most the loads of
    // the NS-2 younger stages remain outstanding (loads retire in order), and
    // its LDS reads of stage it-1 (and, with AQ, of the previous step's codes)
    // have returned once lgkmcnt is 0.  The LDS wait is needed: the compiler
    // moves the MFMAs that consume a step's reads past the next barrier (they
    // touch only registers), so without it those reads can still be queued
    // when the DMA below starts refilling their slot.
    __builtin_amdgcn_s_waitcnt((((NS - 2) * PER_STAGE) & 15) | ((((NS - 2) * PER_STAGE) >> 4) << 14) |
                               (0x7 << 4) | (0x0 << 8));
    // A bare barrier: __syncthreads() adds a workgroup release fence, which
    // waits for every outstanding DMA write to LDS (all NS-1 stages in
    // flight).  Every wave has waited for its own loads of stage `it` and its
    // reads of stage it-1 above, so the barrier alone makes stage `it`
    // complete and slot it-1 free (and the code buffer rewritable).
    asm volatile("s_barrier" ::: "memory");
    issue_stage(it + NS - 1, nxt);
    if constexpr (AQ) {
      quantise_a(cur);
      // the codes are complete (lgkmcnt 0) and visible to every wave
      __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
      asm volatile("s_barrier" ::: "memory");
    }

    // Stages past the K range (issued by the last NS - 1 steps) re-stage the
    // last block; they are never consumed.  Loads are never branched around:
    // at such a merge the compiler's LDS-DMA tracking falls back to waiting
    // for every load.
    float s[NI];
    int ea[NI], eb = 0;  // E8: exponent bytes of this stage's K block
    if constexpr (E8) {
      const int sh = 8 * ((kb0 + it) & 3);
      const uint32_t* w = reinterpret_cast<const uint32_t*>(cur + B_BYTES + A_BYTES);
      eb = (int)((w[SA_BYTES / 4 + wave * 64] >> sh) & 0xFFu);
#pragma unroll
      for (int i = 0; i < NI; ++i) ea[i] = (int)((w[wave * 64 + 16 * i + fr] >> sh) & 0xFFu);
    } else {
      const float sbv = reinterpret_cast<const float*>(cur + B_BYTES + A_BYTES + SA_BYTES)[wave * 64];
      const float* sa_l = AQ ? reinterpret_cast<const float*>(qb + MP * BK)
                             : reinterpret_cast<const float*>(cur + B_BYTES + A_BYTES + wave * 256);
#pragma unroll
      for (int i = 0; i < NI; ++i) s[i] = sa_l[16 * i + fr] * sbv;  // (all 64 slots equal for 128-row A blocks)
    }
    v8i af[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) af[i] = read_frag(AQ ? qb : cur + B_BYTES, 16 * i, off0, off1);
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const v8i bf = read_frag(cur, wave * 16 * F + 16 * f, off0, off1);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if constexpr (E8) {
          acc[f][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], acc[f][i], 0, 0,
                                                                       0, eb, 0, ea[i]);
        } else {
          const v4f part =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], zero, 0, 0, 0, 0, 0, 0);
          acc[f][i] += part * s[i];
        }
      }
    }
  };

  // whole rounds of NS steps (step it + i reads slot i and refills slot
  // i - 1), then the last nk % NS steps after the loop: an exit branch inside
  // the loop body would make the compiler wait for every load at the top of
  // each round
  int it = 0;
  for (; it + NS <= nk; it += NS) {
    static_for<NS>([&](auto tag) {
      constexpr int i = decltype(tag)::value;
      body(it + i, slot(tag), slot(IntTag<(i + NS - 1) % NS>{}));
    });
  }
  static_while<NS - 1>([&](auto tag) {
    constexpr int i = decltype(tag)::value;
    if (it + i >= nk) return false;
    body(it + i, slot(tag), slot(IntTag<(i + NS - 1) % NS>{}));
    return true;
  });
  // drain the re-staged loads past the range before the workgroup exits
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));

  skinny_finish<MP, F>(p, acc, tile, split, n0, lane, wave, s_last);
}

// Optional override for tuning sweeps: DG_SKINNY_SPLITS=<S> (read once).
int forced_splits() {
  static const int v = [] {
    const char* e = getenv("DG_SKINNY_SPLITS");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// B rows per workgroup: 128, or 64 when M > 16 and N gives fewer than 128
// tiles of 128 rows.  64-row tiles re-read A twice as often, but reach a full
// GPU with fewer K splits (less partial traffic, shorter reductions):
// measured on MI355X at M = 64, N = 7168, K = 16384: 39 us (64 rows, 2
// splits) vs 45 us (128 rows, 4 splits); N = 4096, K = 4096: 11.7 vs 18.7 us.
// DG_SKINNY_BN=64|128 overrides it (read once, for tuning sweeps).
int choose_bn(int64_t M, int64_t N) {
  static const int forced = [] {
    const char* e = getenv("DG_SKINNY_BN");
    return e ? atoi(e) : 0;
  }();
  const bool fits64 = (N + 63) / 64 <= kMaxCounters;
  if (forced == 64 && fits64) return 64;
  if (forced == 128) return 128;
  return (M > 16 && (N + 127) / 128 < 128 && fits64) ? 64 : 128;
}

// B rows per workgroup of the kernel that quantises A itself: 128 up to 16
// rows of A (one 16-row block of FP32 A is small next to 16 KB of B); above
// that the plain kernel's rule, except FP32 A of more than 32 rows, which
// takes 64 (with 128 rows its three stages fill all 160 KB of LDS, and the
// kernel measured 178 us against 22 us for BF16 A at 64 x 24576 x 1536).
// DG_SKINNY_BN applies here too.
int fused_bn(int64_t M, int64_t N, bool bf16) {
  if (M <= 16) return 128;
  if (M > 32 && !bf16) return (N + 63) / 64 <= kMaxCounters ? 64 : 128;
  return choose_bn(M, N);
}

int choose_splits(int64_t M, int64_t N, int64_t K) {
  const int bn = choose_bn(M, N);
  const int64_t tiles = (N + bn - 1) / bn;
  const int64_t nkb = K / BK;
  if (forced_splits() > 0) {
    int64_t f = forced_splits();
    f = f > nkb ? nkb : f;
    return (int)(f > kMaxSplits ? kMaxSplits : f);
  }
  // ~one workgroup per CU; more splits only add partial traffic, which grows
  // with M.  Measured on MI355X: M = 64 wants 1 split at N = 24576 (128-row
  // tiles), 2 at N = 7168 and 4 at N = 4096 (64-row tiles); M <= 16 gains
  // from ~two workgroups per CU (8 splits) when N gives few tiles, and loses
  // when it gives many (N = 24576).
  int64_t S = (M <= 16 && tiles < 128) ? 512 / tiles : 256 / tiles;
  S = S < 1 ? 1 : S;
  S = S > (M <= 16 ? 8 : 4) ? (M <= 16 ? 8 : 4) : S;
  S = S > nkb / 3 ? nkb / 3 : S;                // keep >= 3 K blocks (one ring round) per split
  S = S < 1 ? 1 : S;
  return (int)S;
}

// Workspace layout: the arrival counters (kSplitkCounterBytes, at a fixed
// place so that calls of any shape can share one workspace), then the
// partial tiles of the S splits.
void set_split_workspace(SkinnyArgs& p, void* workspace) {
  p.counters = static_cast<int*>(workspace);
  p.partials = workspace ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                    kSplitkCounterBytes)
                         : nullptr;
}

}  // namespace

bool skinny_applies(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 64 && (N + BN - 1) / BN <= kMaxCounters && K >= BK;
}

size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = choose_splits(M, N, K);
  return S > 1 ? kSplitkCounterBytes + (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

template <int AF>
void launch_fused_mp(const SkinnyArgs& p, int mp, int bn, unsigned grid, hipStream_t stream) {
  if (bn == 64) {
    if (mp == 16)
      hipLaunchKernelGGL((gemm_skinny_kernel<16, 1, AF>), dim3(grid), dim3(256), 0, stream, p);
    else if (mp == 32)
      hipLaunchKernelGGL((gemm_skinny_kernel<32, 1, AF>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<64, 1, AF>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (mp == 16)
      hipLaunchKernelGGL((gemm_skinny_kernel<16, 2, AF>), dim3(grid), dim3(256), 0, stream, p);
    else if (mp == 32)
      hipLaunchKernelGGL((gemm_skinny_kernel<32, 2, AF>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<64, 2, AF>), dim3(grid), dim3(256), 0, stream, p);
  }
}

hipError_t launch_gemm_skinny_fused_a(const GemmProblem& q, const void* af, bool bf16,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  SkinnyArgs p;
  p.c = q.c; p.a = nullptr; p.af = af; p.b = q.b; p.sa = nullptr; p.sb = q.sb;
  p.sfa = nullptr; p.sfb = nullptr;
  p.epi = resolved_epilogue(q);
  p.a_block_rows = 1;
  p.M = (int)q.M; p.N = (int)q.N; p.K = (int)q.K;
  p.nkb = (int)(q.K / BK);
  p.sa_stride = p.M;
  p.sb_stride = (int)((q.N + 127) / 128);
  int S = choose_splits(q.M, q.N, q.K);
  // Each step here also encodes A and waits at a second barrier, so short
  // splits cost relatively more: keep >= 5 K blocks per split (measured on
  // MI355X at N = K = 4096: 6 splits 9.4 / 10.5 us at M = 1 / 16, against
  // 10.3 / 12.4 us with the 8 of the plain kernel's rule; N = 7168,
  // K = 16384 keeps 8).  The workspace for the plain rule covers this.
  if (forced_splits() == 0 && S > p.nkb / 5) S = p.nkb / 5 > 1 ? p.nkb / 5 : 1;
  if (workspace == nullptr || workspace_bytes < skinny_workspace_bytes(q.M, q.N, q.K)) S = 1;
  p.S = S;
  set_split_workspace(p, workspace);
  p.part_stride = q.M * q.N;
  p.masked_m = nullptr;
  p.max_m = p.chunks = p.tiles = 0;
  const int mp = q.M <= 16 ? 16 : (q.M <= 32 ? 32 : 64);
  const int bn = fused_bn(q.M, q.N, bf16);
  const unsigned grid = (unsigned)(((q.N + bn - 1) / bn) * S);
  if (bf16) launch_fused_mp<A_BF16>(p, mp, bn, grid, stream);
  else launch_fused_mp<A_F32>(p, mp, bn, grid, stream);
  return hipGetLastError();
}

// Ring depth: 3 slots, except 64-row B tiles with more than 32 rows of A and
// K >= 4096, where a fourth slot (72 KB of LDS: still two workgroups per CU)
// measured faster on MI355X (64 x 7168 x 16384: 37.2 against 39.8 us;
// 64 x 4096 x 4096: 11.9 against 12.1 us; 64 x 24576 x 1536, K = 1536, lost:
// 14.4 against 13.8 us).
template <bool E8>
hipError_t launch_mp(const SkinnyArgs& p, int bn, int64_t M, unsigned grid, hipStream_t stream) {
  if (bn == 64) {
    if (M <= 16)
      hipLaunchKernelGGL((gemm_skinny_kernel<16, 1, A_CODES, E8>), dim3(grid), dim3(256), 0, stream, p);
    else if (M <= 32)
      hipLaunchKernelGGL((gemm_skinny_kernel<32, 1, A_CODES, E8>), dim3(grid), dim3(256), 0, stream, p);
    else if (p.K >= 4096)
      hipLaunchKernelGGL((gemm_skinny_kernel<64, 1, A_CODES, E8, 4>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<64, 1, A_CODES, E8>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (M <= 16)
      hipLaunchKernelGGL((gemm_skinny_kernel<16, 2, A_CODES, E8>), dim3(grid), dim3(256), 0, stream, p);
    else if (M <= 32)
      hipLaunchKernelGGL((gemm_skinny_kernel<32, 2, A_CODES, E8>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<64, 2, A_CODES, E8>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmProblem& q, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  SkinnyArgs p;
  p.c = q.c; p.a = q.a; p.af = nullptr; p.b = q.b; p.sa = q.sa; p.sb = q.sb;
  p.sfa = q.sfa; p.sfb = q.sfb;
  p.epi = resolved_epilogue(q);
  p.a_block_rows = q.a_block_rows;
  p.M = (int)q.M; p.N = (int)q.N; p.K = (int)q.K;
  p.nkb = (int)(q.K / BK);
  p.sa_stride = (int)((q.M + q.a_block_rows - 1) / q.a_block_rows);
  p.sb_stride = (int)((q.N + 127) / 128);
  int S = choose_splits(q.M, q.N, q.K);
  if (workspace == nullptr || workspace_bytes < skinny_workspace_bytes(q.M, q.N, q.K)) S = 1;
  p.S = S;
  set_split_workspace(p, workspace);
  p.part_stride = q.M * q.N;
  p.masked_m = nullptr;
  p.max_m = p.chunks = p.tiles = 0;
  const int bn = choose_bn(q.M, q.N);
  const unsigned grid = (unsigned)(((q.N + bn - 1) / bn) * S);
  return q.sfa ? launch_mp<true>(p, bn, q.M, grid, stream)
               : launch_mp<false>(p, bn, q.M, grid, stream);
}


namespace {

struct MaskedPlan {
  int mp, bn, chunks, tiles, S;
};

// Rows per chunk (the kernel's MP: 16, 32 or 64), B tile rows (as for a
// dense small-M call whose N spans every group and chunk) and splits for the
// masked layout.  Splits: a power of two, at most what gives ~768
// workgroups (two or more per CU hide the weight stream's latency better),
// at most 8, and at least 16 K blocks each.  Measured on MI355X, 8 experts x capacity 32: up projection
// (N 11008, K 4096) 88.6 us with 1 split, 81.3 with 2; down (N 4096,
// K 11008) 85.1 us with 1, 77.0 with 2, 79.5 with 4.
MaskedPlan plan_masked(int num_groups, int64_t max_m, int64_t N, int64_t K) {
  MaskedPlan m;
  m.mp = max_m <= 16 ? 16 : (max_m <= 32 ? 32 : 64);
  m.chunks = (int)((max_m + m.mp - 1) / m.mp);
  const int64_t mc = max_m < m.mp ? max_m : m.mp;
  const int64_t span = N * num_groups * m.chunks;
  m.bn = choose_bn(mc, span);
  m.tiles = (int)((N + m.bn - 1) / m.bn);
  const int64_t wgs = (int64_t)num_groups * m.chunks * m.tiles;
  int64_t S = forced_splits();
  if (S <= 0) {
    const int64_t want = (768 + wgs - 1) / wgs;
    for (S = 1; 2 * S <= want && 2 * S <= (K / BK) / 16; S *= 2) {
    }
  }
  S = S > 8 ? 8 : S;
  S = S > K / BK ? K / BK : S;
  m.S = S < 1 ? 1 : (int)S;
  if (wgs > kMaxCounters) m.S = 1;
  return m;
}

template <int MP, bool E8>
void launch_masked_mp(const SkinnyArgs& p, int bn, unsigned grid, hipStream_t stream) {
  if (bn == 64)
    hipLaunchKernelGGL((gemm_skinny_kernel<MP, 1, A_CODES, E8, 3, true>), dim3(grid), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<MP, 2, A_CODES, E8, 3, true>), dim3(grid), dim3(256), 0,
                       stream, p);
}

template <bool E8>
void launch_masked(const SkinnyArgs& p, int mp, int bn, unsigned grid, hipStream_t stream) {
  if (mp == 16) launch_masked_mp<16, E8>(p, bn, grid, stream);
  else if (mp == 32) launch_masked_mp<32, E8>(p, bn, grid, stream);
  else launch_masked_mp<64, E8>(p, bn, grid, stream);
}

}  // namespace

size_t skinny_masked_workspace_bytes(int num_groups, int64_t max_m, int64_t N, int64_t K) {
  const MaskedPlan m = plan_masked(num_groups, max_m, N, K);
  return m.S > 1 ? kSplitkCounterBytes +
                       (size_t)m.S * (size_t)num_groups * (size_t)max_m * (size_t)N * sizeof(float)
                 : 0;
}

int64_t skinny_masked_grid(int num_groups, int64_t max_m, int64_t N, int64_t K) {
  const MaskedPlan m = plan_masked(num_groups, max_m, N, K);
  return (int64_t)num_groups * m.chunks * m.tiles * m.S;
}

hipError_t launch_gemm_skinny_masked(const GemmProblem& q, const int32_t* masked_m, int64_t max_m,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const MaskedPlan m = plan_masked(q.num_groups, max_m, q.N, q.K);
  SkinnyArgs p;
  p.c = q.c; p.a = q.a; p.af = nullptr; p.b = q.b; p.sa = q.sa; p.sb = q.sb;
  p.sfa = q.sfa; p.sfb = q.sfb;  // UE8M0 words in place of sa / sb, or null
  p.epi = resolved_epilogue(q);
  p.a_block_rows = q.a_block_rows;
  p.M = 0;  // per workgroup: the valid rows of its chunk
  p.N = (int)q.N; p.K = (int)q.K;
  p.nkb = (int)(q.K / BK);
  p.sa_stride = (int)((max_m + q.a_block_rows - 1) / q.a_block_rows);
  p.sb_stride = (int)((q.N + 127) / 128);
  int S = m.S;
  if (workspace == nullptr ||
      workspace_bytes < skinny_masked_workspace_bytes(q.num_groups, max_m, q.N, q.K))
    S = 1;
  p.S = S;
  set_split_workspace(p, workspace);
  p.part_stride = (int64_t)q.num_groups * max_m * q.N;
  p.masked_m = masked_m;
  p.max_m = (int)max_m;
  p.chunks = m.chunks;
  p.tiles = m.tiles;
  const unsigned grid = (unsigned)((int64_t)q.num_groups * m.chunks * m.tiles * S);
  if (q.sfa) launch_masked<true>(p, m.mp, m.bn, grid, stream);
  else launch_masked<false>(p, m.mp, m.bn, grid, stream);
  return hipGetLastError();
}

}  // namespace dg
