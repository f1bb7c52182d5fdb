// Tiled FP8 block-scaled NT GEMM for gfx950 (dense and grouped-M).
//
// What is computed (FP8 block-quantised GEMM page on lpnh.cn, s2.2 and s3.2;
// NT layout and grouped MoE GEMM from the DeepGEMM page on pzsr.cn, s3.1-s3.3):
//   C[m][n] = bf16( sum_kb sa(m,kb) * sb(n,kb) * P_kb[m][n] ),
//   P_kb[m][n] = sum_{k in 128-wide block kb} A[m][k] * B[n][k]
// with the E4M3 products summed in FP32 by the matrix cores and promoted into
// FP32 accumulators once per 128-wide K block.
//
// gfx950 mapping
//  * One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-wide K block of a
//    16x16 output sub-tile, so the per-block partial P_kb never needs more
//    than 4 transient VGPRs: it is produced with a zero accumulator and
//    immediately folded into the FP32 accumulator with one FMA per element
//    (acc += P_kb * sa*sb).  The MFMA operands are swapped (B rows feed the
//    instruction's first operand) so each lane ends up owning 4 consecutive
//    output columns of one row: one scale per lane and sub-tile row, and
//    8-byte BF16 stores.
//  * Workgroup tile BM x 256, K step 128; waves own 64 x 128 sub-tiles
//    (4 x 8 MFMA tiles, 128 accumulator VGPRs).  BM = 256 -> 8 waves.
//  * Global -> LDS staging with global_load_lds_dwordx4 (no VGPR round trip),
//    two LDS stages held in two distinct __shared__ arrays so that the
//    compiler's LDS-DMA wait tracking can tell the stages apart.
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//    c ^ x(r), x(r) = ((r & 3) << 1) ^ ((r >> 2) & 1).  This permutation was
//    chosen by measurement (LDS bank-conflict counters on gfx950 over the
//    exact fragment-read pattern, 16 rows x one chunk per 16-lane group, all
//    four groups at different chunks of the same rows): it is conflict-free,
//    while the XOR swizzles that merely give the 16 lanes distinct banks of a
//    64 x 4-byte bank map are not.  The DMA writes stay linear (the
//    permutation is applied to the global source addresses), so every 8
//    consecutive lanes still fetch one full 128-byte row segment.
//  * Workgroup ids are remapped so that each XCD (ids round-robin over 8
//    XCDs) works on a contiguous patch of tiles that shares A and B panels in
//    its own L2 (see map_tile).
#include "dg_device.hpp"
#include "dg_internal.hpp"

#include <stdlib.h>

namespace dg {
namespace {

constexpr int BN = 256;
constexpr int BK = 128;

// s_waitcnt immediate: vmcnt(4), expcnt and lgkmcnt left at their maxima.
constexpr int kVmcnt4 = 4 | (7 << 4) | (15 << 8);

struct TiledArgs {
  uint16_t* c;
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  const uint32_t* sfa;  // UE8M0 variant: packed exponent words instead of sa / sb
  const uint32_t* sfb;
  const int32_t* m_indices;
  const int64_t* k_offsets;  // K-grouped: group g covers K [k_offsets[g], k_offsets[g+1])
  int num_groups;
  Epilogue epi;  // dense only (grouped: none)
  int M, N, K;
  int nkb;        // K / 128
  int sa_stride;  // ceil(M / a_block_rows)
  int sb_stride;  // ceil(N / 128)
  int tiles_m, tiles_n;
  int group_m;
  int grouped_n_major;  // grouped tile order: N-tile-major instead of row-block-major
};

__device__ __forceinline__ int lds_swz(int r) { return ((r & 3) << 1) ^ ((r >> 2) & 1); }

// Stage one BK-wide slice of a ROWS x 128-byte operand tile into LDS.
// Wave w issues ITERS instructions; instruction j fills LDS bytes
// [cb*1024, cb*1024 + 1024) with cb = j*NW + w, i.e. rows cb*8 .. cb*8+7.
template <int ROWS, int NW>
struct TileLoader {
  static constexpr int ITERS = ROWS / 8 / NW;
  uint32_t off[ITERS];  // byte offset of this lane's source chunk at kb = 0

  __device__ __forceinline__ void init(int wave, int lane, int row0, int rows_valid, int K) {
#pragma unroll
    for (int j = 0; j < ITERS; ++j) {
      const int cb = j * NW + wave;
      const int r = cb * 8 + (lane >> 3);
      const int logical = (lane & 7) ^ lds_swz(r);
      int gr = row0 + r;
      gr = gr < rows_valid ? gr : rows_valid - 1;  // clamp: rows past the edge only feed
                                                    // outputs that are never stored
      off[j] = (uint32_t)gr * (uint32_t)K + (uint32_t)(logical * 16);
    }
  }

  __device__ __forceinline__ void issue_one(const uint8_t* base, uint8_t* lds, int wave, int kb,
                                            int j) const {
    const int cb = j * NW + wave;
    __builtin_amdgcn_global_load_lds(
        (const void*)(base + off[j] + (uint32_t)kb * BK),
        (__attribute__((address_space(3))) void*)(lds + cb * 1024), 16, 0, 0);
  }

  // base + koff is the (uniform) start of the K block; the empty asm hides the
  // lane offset from loop strength reduction, which would otherwise keep one
  // pointer per (instruction, unrolled step) live
  __device__ __forceinline__ void issue_at(const uint8_t* base, uint32_t koff, uint8_t* lds,
                                           int wave, int j) const {
    const int cb = j * NW + wave;
    uint32_t o = off[j];
    asm volatile("" : "+v"(o));
    __builtin_amdgcn_global_load_lds((const void*)(base + (o + koff)),
                                     (__attribute__((address_space(3))) void*)(lds + cb * 1024),
                                     16, 0, 0);
  }

  __device__ __forceinline__ void issue(const uint8_t* base, uint8_t* lds, int wave, int kb) const {
#pragma unroll
    for (int j = 0; j < ITERS; ++j) issue_one(base, lds, wave, kb, j);
  }
};

__device__ __forceinline__ v8i read_frag(const uint8_t* lds, int row_base, int off0, int off1) {
  const v4i lo = *reinterpret_cast<const v4i*>(lds + row_base * 128 + off0);
  const v4i hi = *reinterpret_cast<const v4i*>(lds + row_base * 128 + off1);
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Workgroup ids are dealt round-robin to the 8 XCDs (id % 8), each with its
// own L2.  The id is first turned into a position L in a tile order such that
// every XCD gets a contiguous run of L (a bijection for any tile count), then
// L is mapped to a tile.  Dense: groups of group_m tile-rows swept along N,
// so concurrently running tiles share A and B panels.  Grouped: row-block-
// major, so an XCD works through all N tiles of two or three 128-row blocks
// (their A rows stay in its L2) and the row tiles of one expert follow each
// other, the second pass over the expert's weights finding them in the
// Infinity Cache.  Measured on MI355X (8 experts, 1024 tokens top-2): up
// projection 187 -> 159 us, down 159 -> 155 us against the N-tile-major order
// (p.grouped_n_major, kept for tuning).
__device__ __forceinline__ void map_tile(const TiledArgs& p, bool grouped, int& tm, int& tn,
                                         int groups = 1, int* kgroup = nullptr) {
  const int bid = blockIdx.x;
  const int per_g = p.tiles_m * p.tiles_n;
  const int total = per_g * groups;
  const int x = bid & 7, per = total >> 3, extra = total & 7;
  int L = x * per + min(x, extra) + (bid >> 3);
  if (kgroup) {  // K-grouped: consecutive positions stay within one group's tiles
    *kgroup = L / per_g;
    L -= *kgroup * per_g;
  }
  if (grouped) {
    if (p.grouped_n_major) {
      tn = L / p.tiles_m;
      tm = L - tn * p.tiles_m;
    } else {
      tm = L / p.tiles_n;
      tn = L - tm * p.tiles_n;
    }
    return;
  }
  const int per_group = p.group_m * p.tiles_n;
  const int group = L / per_group;
  const int first_m = group * p.group_m;
  const int gsz = min(p.tiles_m - first_m, p.group_m);
  const int rem = L - group * per_group;
  tm = first_m + rem % gsz;
  tn = rem / gsz;
}

// Grouped tiles are indexed by 128-row block.  Every block carries one expert
// id (rows of an expert are contiguous and padded to 128).  The blocks of one
// expert are paired: the first block of each pair computes a 256-row tile,
// the second has nothing to do, and an odd block left at the end of an
// expert's run computes 128 rows (the loads and MFMAs of the other half are
// spent on clamped rows that are never stored).  A block whose first row is
// padding (id -1) is all padding: its workgroup writes zeros.  Returns false
// when the workgroup has nothing more to do.
__device__ __forceinline__ bool grouped_tile(const TiledArgs& p, int blk, int n0, int lane,
                                             int& m0, int& rows_end, const uint8_t*& bbase,
                                             const float*& sbbase, const uint32_t*& sfbbase) {
  m0 = blk * 128;
  const int g = p.m_indices[m0];
  if (g < 0 || g >= p.num_groups) {
    // the block's output columns (half of the tile's with SwiGLU), 4 per store
    const bool glu = p.epi.act == EPI_SWIGLU;
    const int64_t ldc = p.epi.ldc;
    const int oc0 = glu ? n0 / 2 : n0;
    constexpr int Q = BN / 4;  // 4-column groups per row (SwiGLU uses the first half)
    for (int idx = threadIdx.x; idx < 128 * Q; idx += blockDim.x) {
      const int r = idx / Q;
      const int cc = (idx % Q) * 4;
      if ((!glu || cc < BN / 2) && oc0 + cc < ldc)
        *reinterpret_cast<uint2*>(p.c + (int64_t)(m0 + r) * ldc + oc0 + cc) = make_uint2(0, 0);
    }
    return false;
  }
  // first block of the run of blocks with id g that ends at blk: each lane
  // looks at one earlier block, 64 blocks per round
  int start = 0;
  for (int base = blk;; base -= 64) {
    const int bb = base - 1 - lane;
    const bool differs = bb < 0 || p.m_indices[(int64_t)bb * 128] != g;
    const unsigned long long mask = __ballot(differs);
    if (mask != 0ull) {
      start = base - (__ffsll(mask) - 1);
      break;
    }
  }
  if ((blk - start) & 1) return false;  // covered by the tile of the previous block
  const int nblk = p.M / 128;
  const bool pair = blk + 1 < nblk && p.m_indices[(int64_t)(blk + 1) * 128] == g;
  rows_end = m0 + (pair ? 256 : 128);
  bbase += (int64_t)g * p.N * p.K;
  sbbase += (int64_t)g * p.nkb * p.sb_stride;
  sfbbase += (int64_t)g * ((p.nkb + 3) / 4) * p.sb_stride;  // UE8M0: four K blocks per word
  return true;
}

// Grouped epilogue straight from the MFMA layout (lane: 4 consecutive
// columns of one row per 16 x 16 sub-tile): the fused epilogue on real rows,
// zeros on padding rows (id -1; with SwiGLU the row's half-width output).
__device__ __forceinline__ void grouped_store(const TiledArgs& p, const v4f (&acc)[4][8], int m0,
                                              int nw0, int mw0, int rows_end, int lane) {
  const int fr = lane & 15;
  with_epilogue(p.epi, [&](auto act, auto res) {
    constexpr int ACT = decltype(act)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mw0 + 16 * i + fr;
      if (m >= rows_end) continue;
      const bool zero_row = p.m_indices[m] < 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = nw0 + 16 * j + 4 * (lane >> 4);
        if (n >= p.N) continue;
        if (zero_row) {
          if (ACT == EPI_SWIGLU)
            *reinterpret_cast<uint32_t*>(p.c + (int64_t)m * p.epi.ldc + (n >> 1)) = 0u;
          else
            *reinterpret_cast<uint2*>(p.c + (int64_t)m * p.epi.ldc + n) = make_uint2(0, 0);
        } else {
          const float t[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          store4<ACT, decltype(res)::value != 0>(p.c, m, n, t, p.epi);
        }
      }
    }
  });
}

// E8: power-of-two (UE8M0) scales (DeepGEMM page on pzsr.cn, s3.1), four K
// blocks per 32-bit word.  The scaled MFMA applies them itself -- each lane
// passes the exponent byte of the row it feeds (one byte per 32 products of
// that row; a 128-K block uses the same byte for all four) -- so the
// accumulators chain through K with no partials and no promotion FMAs.
// KG: K-grouped (DeepGEMM page on pzsr.cn, s3.2: grouping along K, the MoE
// weight-gradient layout): the grid covers num_groups x the output tiles;
// group g runs the K blocks [k_offsets[g] / 128, k_offsets[g+1] / 128) and
// writes C + g * M * N (an empty range writes zeros).
template <int BM, int A_BLK, bool GROUPED, bool E8 = false, bool KG = false>
__global__ void __launch_bounds__(BM * BN / 128)
gemm_tiled_kernel(TiledArgs p) {
  constexpr int WM = BM / 64;
  constexpr int NW = WM * (BN / 128);
  constexpr int A_BYTES = BM * BK;
  constexpr int STAGE = A_BYTES + BN * BK;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = wave % WM;
  const int wn = wave / WM;

  int tm, tn, kgroup = 0;
  map_tile(p, GROUPED, tm, tn, KG ? p.num_groups : 1, KG ? &kgroup : nullptr);
  const int n0 = tn * BN;
  int m0 = tm * BM;
  int rows_end = p.M;  // rows [m0, rows_end) are stored
  int kb_begin = 0, kb_end = p.nkb;
  uint16_t* cbase = p.c;
  if (KG) {
    // clamped into [0, nkb]: offsets that break the contract give wrong sums,
    // never reads outside A, B or the scales
    int64_t k0 = p.k_offsets[kgroup] / BK, k1 = p.k_offsets[kgroup + 1] / BK;
    k0 = k0 < 0 ? 0 : (k0 > p.nkb ? p.nkb : k0);
    k1 = k1 < k0 ? k0 : (k1 > p.nkb ? p.nkb : k1);
    kb_begin = (int)k0;
    kb_end = (int)k1;
    cbase += (int64_t)kgroup * p.M * p.N;
  }

  const uint8_t* bbase = p.b;
  const float* sbbase = p.sb;
  const uint32_t* sfbbase = p.sfb;  // UE8M0 B exponents (the expert's, when grouped)
  if (GROUPED) {
    if (!grouped_tile(p, tm, n0, lane, m0, rows_end, bbase, sbbase, sfbbase)) return;
  }

  TileLoader<BM, NW> lda;
  TileLoader<BN, NW> ldb;
  lda.init(wave, lane, m0, rows_end, p.K);
  ldb.init(wave, lane, n0, p.N, p.K);

  // fragment read offsets (constant per lane: the swizzle depends on r % 8 only)
  const int fr = lane & 15;
  const int off0 = fr * 128 + (((2 * (lane >> 4)) ^ lds_swz(fr)) * 16);
  const int off1 = fr * 128 + (((2 * (lane >> 4) + 1) ^ lds_swz(fr)) * 16);

  // scale indices
  int sa_idx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + wm * 64 + 16 * i + fr;
    if (A_BLK == 1) {
      sa_idx[i] = m < rows_end ? m : rows_end - 1;
    } else {
      int rb = (m0 + wm * 64) / 128;
      sa_idx[i] = rb < p.sa_stride ? rb : p.sa_stride - 1;
    }
  }
  int nb = (n0 + wn * 128) / 128;
  nb = nb < p.sb_stride ? nb : p.sb_stride - 1;

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  float sa_cur[4], sa_nxt[4];
  float sb_cur, sb_nxt;
  int ea_cur[4], ea_nxt[4], eb_cur = 0, eb_nxt = 0;  // E8: exponent bytes (bits 7:0)
  if constexpr (E8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ea_cur[i] = (int)(p.sfa[sa_idx[i]] & 0xFFu);
    eb_cur = (int)(sfbbase[nb] & 0xFFu);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) sa_cur[i] = p.sa[(int64_t)kb_begin * p.sa_stride + sa_idx[i]];
    sb_cur = sbbase[(int64_t)kb_begin * p.sb_stride + nb];
  }

  if (kb_end > kb_begin) {  // uniform per workgroup (false only for an empty K group)
    lda.issue(p.a, lds0, wave, kb_begin);
    ldb.issue(bbase, lds0 + A_BYTES, wave, kb_begin);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  auto step = [&](const uint8_t* cur, uint8_t* nxt, int kb) {
    // The last step re-stages the final K slice into the idle buffer so the
    // body stays one basic block (the scheduling hints below need that).
    const int kn = kb + 1 < kb_end ? kb + 1 : kb;
    float s[4];
    if constexpr (E8) {
      const int w = kn >> 2, sh = 8 * (kn & 3);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ea_nxt[i] = (int)((p.sfa[(int64_t)w * p.sa_stride + sa_idx[i]] >> sh) & 0xFFu);
      eb_nxt = (int)((sfbbase[(int64_t)w * p.sb_stride + nb] >> sh) & 0xFFu);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) sa_nxt[i] = p.sa[(int64_t)kn * p.sa_stride + sa_idx[i]];
      sb_nxt = sbbase[(int64_t)kn * p.sb_stride + nb];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = sa_cur[i] * sb_cur;
    }

    v8i af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = read_frag(cur, wm * 64 + 16 * i, off0, off1);
    v8i bf[2];
    bf[0] = read_frag(cur + A_BYTES, wn * 128, off0, off1);
    // 32 MFMAs in (j, i) order.  The 4 promotion FMAs of MFMA t are issued
    // after MFMA t+1, so they overlap the matrix core instead of stalling on
    // its result; the next B fragment is read right after the first MFMA of
    // each group of four; the DMA instructions staging the next K step are
    // spread one per two MFMAs over the first half (issued back to back they
    // stall the wave on a full memory queue before its MFMAs can start).
    // The fences pin this order against the scheduler, which otherwise
    // hoists all MFMAs and parks 32 partials in registers.
    constexpr int IA = TileLoader<BM, NW>::ITERS, IB = TileLoader<BN, NW>::ITERS;
    static_assert(2 * (IA + IB) <= 32, "DMA issue slots");
    v4f part[2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int j = t >> 2, i = t & 3;
      if constexpr (E8)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bf[j & 1], af[i], acc[i][j], 0, 0, 0, eb_cur, 0, ea_cur[i]);
      else
        part[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j & 1], af[i], zero, 0,
                                                                       0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if ((t & 1) == 0 && (t >> 1) < IA + IB) {
        const int q = t >> 1;
        if (q < IA)
          lda.issue_one(p.a, nxt, wave, kn, q);
        else
          ldb.issue_one(bbase, nxt + A_BYTES, wave, kn, q - IA);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 0 && j < 7) {
        bf[(j + 1) & 1] = read_frag(cur + A_BYTES, wn * 128 + 16 * (j + 1), off0, off1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!E8 && t > 0) {
        const int tp = t - 1, jp = tp >> 2, ip = tp & 3;
        acc[ip][jp] += part[tp & 1] * s[ip];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (E8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ea_cur[i] = ea_nxt[i];
      eb_cur = eb_nxt;
    } else {
      acc[3][7] += part[1] * s[3];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa_cur[i] = sa_nxt[i];
      sb_cur = sb_nxt;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  for (int kb = kb_begin; kb < kb_end; kb += 2) {
    step(lds0, lds1, kb);
    if (kb + 1 < kb_end) step(lds1, lds0, kb + 1);
  }

  if constexpr (GROUPED) {
    grouped_store(p, acc, m0, n0 + wn * 128, wm * 64, rows_end, lane);
  } else {
    // The finished tile leaves through LDS.  Stored straight from the MFMA
    // layout, each store instruction writes 32 bytes into each of 16 rows;
    // when C does not fit in the Infinity Cache those scattered pieces cap
    // the write rate far below HBM's.  Staged, every instruction writes whole
    // 512-byte row segments.  Staged row r (BF16, ocols per row) sits in lds0
    // (r < 128) or lds1 at (r % 128) * rowb, its 16-byte chunk c at chunk
    // c ^ (r % chunks) (the 16 rows of one MFMA-layout write hit distinct
    // banks; the row-wise reads are conflict-free either way).  The K loop
    // ended with a barrier after its last LDS read and DMA.
    const bool glu = p.epi.act == EPI_SWIGLU;
    const int rowb = glu ? BN : 2 * BN;  // bytes per staged row
    const int chunks = rowb / 16;
    with_epilogue(p.epi, [&](auto act, auto res) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + 16 * i + fr;
        const int m = m0 + r < rows_end ? m0 + r : rows_end - 1;  // (row not stored)
        uint8_t* row = (r < 128 ? lds0 : lds1) + (r & 127) * rowb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int nl = wn * 128 + 16 * j + 4 * (lane >> 4);
          const int n = n0 + nl < p.N ? n0 + nl : p.N - 4;  // (column not stored)
          const float t[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          uint2 v;
          const int cnt =
              epilogue4<decltype(act)::value, decltype(res)::value != 0>(m, n, t, p.epi, v);
          const int ob = (cnt == 2 ? nl : 2 * nl);  // byte offset of the first output column
          uint8_t* dst = row + ((((ob >> 4) ^ (r % chunks)) << 4) | (ob & 15));
          if (cnt == 2)
            *reinterpret_cast<uint32_t*>(dst) = v.x;
          else
            *reinterpret_cast<uint2*>(dst) = v;
        }
      }
    });
    __syncthreads();
    const int64_t ldc = p.epi.ldc;
    const int64_t oc0 = glu ? n0 / 2 : n0;  // first output column of the tile
    const bool wide = (ldc & 7) == 0;       // 16-byte stores stay aligned
    for (int q = threadIdx.x; q < BM * chunks; q += BM * BN / 128) {
      const int r = q / chunks, cc = q - r * chunks;
      const int64_t m = m0 + r;
      const int64_t col = oc0 + 8 * cc;
      if (m >= rows_end || col >= ldc) continue;
      const uint4 v = *reinterpret_cast<const uint4*>((r < 128 ? lds0 : lds1) + (r & 127) * rowb +
                                                       ((cc ^ (r % chunks)) << 4));
      uint16_t* g = cbase + m * ldc + col;
      if (wide && col + 8 <= ldc) {
        *reinterpret_cast<uint4*>(g) = v;
      } else {
        *reinterpret_cast<uint2*>(g) = make_uint2(v.x, v.y);
        if (col + 8 <= ldc) *reinterpret_cast<uint2*>(g + 4) = make_uint2(v.z, v.w);
      }
    }
  }
}

// 256 x 256 tile with a five-slot LDS ring of half stages, for operands that
// stream from HBM (grouped MoE weights), where one stage of lookahead does not
// cover the memory latency.
//
// A half stage is one 32 KB operand slice (A or B, 256 rows x 128 K bytes);
// the 160 KB of LDS hold five of them.  Step k reads A_k and B_k from slots
// 2k+1 mod 5 and 2k mod 5 while the DMA for A_{k+1}, then B_{k+2}, streams
// into the two slots that step k-1 released, one DMA instruction per four
// MFMAs.  B (the weights, from HBM) is thus requested about one and a half
// steps before it is read, A (re-read by many tiles, mostly from L2) about
// one step before.  At the top of step k every slice except the most recent
// (B_{k+1}) must have landed: s_waitcnt vmcnt(4), then one barrier, which
// also certifies that all waves have finished reading the slots about to be
// refilled.
template <int A_BLK, bool GROUPED>
__global__ void __launch_bounds__(512)
gemm_ring_kernel(TiledArgs p) {
  constexpr int BM = 256;
  constexpr int WM = 4;
  constexpr int NW = 8;
  constexpr int HALF = 256 * BK;
  __shared__ __attribute__((aligned(1024))) uint8_t r0[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r2[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r3[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r4[HALF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = wave % WM;
  const int wn = wave / WM;

  int tm, tn;
  map_tile(p, GROUPED, tm, tn);
  const int n0 = tn * BN;
  int m0 = tm * BM;
  int rows_end = p.M;
  const uint8_t* bbase = p.b;
  const float* sbbase = p.sb;
  const uint32_t* sfbbase = p.sfb;  // UE8M0 B exponents (the expert's, when grouped)
  if (GROUPED) {
    if (!grouped_tile(p, tm, n0, lane, m0, rows_end, bbase, sbbase, sfbbase)) return;
  }

  TileLoader<BM, NW> lda;
  TileLoader<BN, NW> ldb;
  lda.init(wave, lane, m0, rows_end, p.K);
  ldb.init(wave, lane, n0, p.N, p.K);

  const int fr = lane & 15;
  const int off0 = fr * 128 + (((2 * (lane >> 4)) ^ lds_swz(fr)) * 16);
  const int off1 = fr * 128 + (((2 * (lane >> 4) + 1) ^ lds_swz(fr)) * 16);

  int sa_idx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + wm * 64 + 16 * i + fr;
    if (A_BLK == 1) {
      sa_idx[i] = m < rows_end ? m : rows_end - 1;
    } else {
      int rb = (m0 + wm * 64) / 128;
      sa_idx[i] = rb < p.sa_stride ? rb : p.sa_stride - 1;
    }
  }
  int nb = (n0 + wn * 128) / 128;
  nb = nb < p.sb_stride ? nb : p.sb_stride - 1;
  const int last = p.nkb - 1;

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // The scales of block k are loaded during step k-1 (block 0 here) and their
  // products formed at the top of step k, after the wait that covers them.
  float sa_nxt[4];
  float sb_nxt = sbbase[nb];
#pragma unroll
  for (int i = 0; i < 4; ++i) sa_nxt[i] = p.sa[sa_idx[i]];

  // prologue: A_0, B_0, B_1 (B_1 re-reads block 0 when K has one block)
  lda.issue(p.a, r1, wave, 0);
  ldb.issue(bbase, r0, wave, 0);
  ldb.issue(bbase, r2, wave, last > 0 ? 1 : 0);

  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  auto step = [&](const uint8_t* a_l, const uint8_t* b_l, uint8_t* wa, uint8_t* wb, int kb) {
    __builtin_amdgcn_s_waitcnt(kVmcnt4);
    asm volatile("s_barrier" ::: "memory");
    float s_cur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s_cur[i] = sa_nxt[i] * sb_nxt;
    // uniform per-step block indices (readfirstlane keeps the compiler from
    // deriving one pointer induction variable per unrolled step)
    const int k1 = __builtin_amdgcn_readfirstlane(kb + 1 < last ? kb + 1 : last);
    const int k2 = __builtin_amdgcn_readfirstlane(kb + 2 < last ? kb + 2 : last);
    const float* sa_row = p.sa + (int64_t)k1 * p.sa_stride;
    const float* sb_row = sbbase + (int64_t)k1 * p.sb_stride;
    const uint32_t kb1 = (uint32_t)k1 * BK, kb2 = (uint32_t)k2 * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o = (uint32_t)sa_idx[i] * 4u;
      asm volatile("" : "+v"(o));
      sa_nxt[i] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sa_row) + o);
    }
    sb_nxt = sb_row[nb];

    v8i af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = read_frag(a_l, wm * 64 + 16 * i, off0, off1);
    v8i bf[2];
    bf[0] = read_frag(b_l, wn * 128, off0, off1);
    v4f part[2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int j = t >> 2, i = t & 3;
      part[t & 1] =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j & 1], af[i], zero, 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if ((t & 3) == 1) {
        const int q = t >> 2;  // A_{k+1} parts 0..3, then B_{k+2} parts 0..3
        if (q < 4)
          lda.issue_at(p.a, kb1, wa, wave, q);
        else
          ldb.issue_at(bbase, kb2, wb, wave, q - 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 0 && j < 7) {
        bf[(j + 1) & 1] = read_frag(b_l, wn * 128 + 16 * (j + 1), off0, off1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t > 0) {
        const int tp = t - 1, jp = tp >> 2, ip = tp & 3;
        acc[ip][jp] += part[tp & 1] * s_cur[ip];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    acc[3][7] += part[1] * s_cur[3];
  };

  // A_k sits in slot 2k+1 mod 5 and B_k in 2k mod 5; step k fills the two
  // slots step k-1 read with A_{k+1} and B_{k+2}.  The pattern repeats every
  // five steps
  int kb = 0;
  for (; kb + 5 <= p.nkb; kb += 5) {
    step(r1, r0, r3, r4, kb);
    step(r3, r2, r0, r1, kb + 1);
    step(r0, r4, r2, r3, kb + 2);
    step(r2, r1, r4, r0, kb + 3);
    step(r4, r3, r1, r2, kb + 4);
  }
  if (kb < p.nkb) step(r1, r0, r3, r4, kb);
  if (kb + 1 < p.nkb) step(r3, r2, r0, r1, kb + 1);
  if (kb + 2 < p.nkb) step(r0, r4, r2, r3, kb + 2);
  if (kb + 3 < p.nkb) step(r2, r1, r4, r0, kb + 3);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if constexpr (GROUPED) {
    grouped_store(p, acc, m0, n0 + wn * 128, wm * 64, rows_end, lane);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + 16 * i + fr;
      if (m >= rows_end) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = n0 + wn * 128 + 16 * j + 4 * (lane >> 4);
        if (n < p.N) {
          const float t[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          store4<EPI_NONE, false>(p.c, m, n, t, p.epi);  // dense ring: no epilogue
        }
      }
    }
  }
}

// Tile rows per band of the dense tile order (see map_tile); DG_GROUP_M
// overrides it (read once, for tuning sweeps).
int group_m() {
  static const int v = [] {
    const char* e = getenv("DG_GROUP_M");
    const int g = e ? atoi(e) : 0;
    return g > 0 ? g : 4;
  }();
  return v;
}

// DG_GROUPED_ORDER=n selects the N-tile-major grouped tile order (read
// once, for tuning sweeps).
int grouped_n_major() {
  static const int v = [] {
    const char* e = getenv("DG_GROUPED_ORDER");
    return e && e[0] == 'n' ? 1 : 0;
  }();
  return v;
}

template <bool RING, int A_BLK, bool GROUPED, bool E8 = false, bool KG = false>
hipError_t launch_one(const GemmProblem& q, hipStream_t stream) {
  static_assert(!(E8 && RING), "UE8M0 scales: two-stage kernel only");
  static_assert(!(KG && (RING || GROUPED || E8)), "K-grouped: dense two-stage kernel only");
  TiledArgs p;
  p.c = q.c; p.a = q.a; p.b = q.b; p.sa = q.sa; p.sb = q.sb;
  p.sfa = q.sfa; p.sfb = q.sfb;
  p.epi = resolved_epilogue(q);
  p.m_indices = q.m_indices; p.num_groups = q.num_groups;
  p.k_offsets = q.k_offsets;
  p.M = (int)q.M; p.N = (int)q.N; p.K = (int)q.K;
  p.nkb = (int)(q.K / BK);
  p.sa_stride = (int)((q.M + q.a_block_rows - 1) / q.a_block_rows);
  p.sb_stride = (int)((q.N + 127) / 128);
  p.tiles_m = GROUPED ? (int)(q.M / 128) : (int)((q.M + 255) / 256);
  p.tiles_n = (int)((q.N + BN - 1) / BN);
  p.group_m = group_m();
  p.grouped_n_major = grouped_n_major();
  const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n) * (KG ? (unsigned)q.num_groups : 1u);
  if constexpr (RING)
    hipLaunchKernelGGL((gemm_ring_kernel<A_BLK, GROUPED>), dim3(grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<256, A_BLK, GROUPED, E8, KG>), dim3(grid), dim3(512), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace

// Kernel choice (DG_TILED=pair|ring overrides it, read once, for tuning): the
// two-stage kernel for dense operands, which mostly hit in L2; the ring for
// grouped weights, which stream from HBM.
hipError_t launch_gemm_tiled(const GemmProblem& q, bool grouped, hipStream_t stream) {
  static const int forced = [] {
    const char* e = getenv("DG_TILED");
    return e ? (e[0] == 'p' ? 1 : (e[0] == 'r' ? 2 : 0)) : 0;
  }();
  // (the ring kernel has no epilogue: a dense call with one stays on the pair kernel)
  const bool plain = q.epi.act == EPI_NONE && q.epi.res == nullptr;
  const bool ring = (forced ? forced == 2 : grouped) && (grouped || plain);
  if (grouped) {
    if (ring)
      return q.a_block_rows == 1 ? launch_one<true, 1, true>(q, stream)
                                 : launch_one<true, 128, true>(q, stream);
    return q.a_block_rows == 1 ? launch_one<false, 1, true>(q, stream)
                               : launch_one<false, 128, true>(q, stream);
  }
  if (ring)
    return q.a_block_rows == 1 ? launch_one<true, 1, false>(q, stream)
                               : launch_one<true, 128, false>(q, stream);
  return q.a_block_rows == 1 ? launch_one<false, 1, false>(q, stream)
                             : launch_one<false, 128, false>(q, stream);
}

hipError_t launch_gemm_tiled_kgrouped(const GemmProblem& q, hipStream_t stream) {
  return q.a_block_rows == 1 ? launch_one<false, 1, false, false, true>(q, stream)
                             : launch_one<false, 128, false, false, true>(q, stream);
}

// Grouped with UE8M0 scales: the two-stage kernel (the grouped ring kernel
// has no UE8M0 form; with the exponent registers on top of its five-slot
// pipeline state it would not fit the register file without spills).
hipError_t launch_gemm_tiled_grouped_ue8m0(const GemmProblem& q, hipStream_t stream) {
  return q.a_block_rows == 1 ? launch_one<false, 1, true, true>(q, stream)
                             : launch_one<false, 128, true, true>(q, stream);
}

hipError_t launch_gemm_tiled_ue8m0(const GemmProblem& q, hipStream_t stream) {
  return q.a_block_rows == 1 ? launch_one<false, 1, false, true>(q, stream)
                             : launch_one<false, 128, false, true>(q, stream);
}

}  // namespace dg
