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

#include <limits.h>
#include <stdlib.h>

namespace dg {
namespace {

constexpr int BN = 256;
constexpr int BK = 128;

typedef unsigned v4u __attribute__((ext_vector_type(4)));

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

// Zeros into the 128 rows of a padding block from m0 and the output columns
// of the 256-column tile at n0 (half of them with SwiGLU), 4 per store, by
// all threads of the workgroup.
__device__ __forceinline__ void zero_block(const TiledArgs& p, int m0, int n0) {
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
    zero_block(p, m0, n0);
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
struct Ring {
  uint8_t *r0, *r1, *r2, *r3, *r4;
};

// The operand slices, scale positions and fragment offsets of one 256 x 256
// tile at rows m0 (rows from rows_end on are clamped) and columns n0.
struct RingTile {
  TileLoader<256, 8> lda, ldb;
  const uint8_t* bbase;
  const float* sbbase;
  int sa_idx[4];
  int nb;
};

template <int A_BLK>
__device__ __forceinline__ void ring_tile_init(const TiledArgs& p, RingTile& t, int m0, int rows_end,
                                               int n0, int wave, int lane) {
  const int wm = wave % 4, wn = wave / 4, fr = lane & 15;
  t.lda.init(wave, lane, m0, rows_end, p.K);
  t.ldb.init(wave, lane, n0, p.N, p.K);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + wm * 64 + 16 * i + fr;
    if (A_BLK == 1) {
      t.sa_idx[i] = m < rows_end ? m : rows_end - 1;
    } else {
      int rb = (m0 + wm * 64) / 128;
      t.sa_idx[i] = rb < p.sa_stride ? rb : p.sa_stride - 1;
    }
  }
  int nb = (n0 + wn * 128) / 128;
  t.nb = nb < p.sb_stride ? nb : p.sb_stride - 1;
}

// Adds the K blocks [k0, k1) (k1 > k0) of the tile into acc.  Returns with
// every DMA of this wave complete; the LDS reads of other waves may still be
// in flight.
__device__ __forceinline__ void ring_run(const TiledArgs& p, const Ring& R, const RingTile& t,
                                         int k0, int k1, int wave, int lane,
                                         v4f (&acc)[4][8]) {
  const int wm = wave % 4, wn = wave / 4, fr = lane & 15;
  const int off0 = fr * 128 + (((2 * (lane >> 4)) ^ lds_swz(fr)) * 16);
  const int off1 = fr * 128 + (((2 * (lane >> 4) + 1) ^ lds_swz(fr)) * 16);
  const int last = k1 - 1;

  // The scales of block k are loaded during step k-1 (block k0 here) and their
  // products formed at the top of step k, after the wait that covers them.
  float sa_nxt[4];
  float sb_nxt = t.sbbase[(int64_t)k0 * p.sb_stride + t.nb];
#pragma unroll
  for (int i = 0; i < 4; ++i) sa_nxt[i] = p.sa[(int64_t)k0 * p.sa_stride + t.sa_idx[i]];

  // prologue: A_k0, B_k0, B_k0+1 (B_k0+1 re-reads block k0 when the range has one block)
  t.lda.issue(p.a, R.r1, wave, k0);
  t.ldb.issue(t.bbase, R.r0, wave, k0);
  t.ldb.issue(t.bbase, R.r2, wave, k0 < last ? k0 + 1 : k0);

  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  auto step = [&](const uint8_t* a_l, const uint8_t* b_l, uint8_t* wa, uint8_t* wb, int kb) {
    __builtin_amdgcn_s_waitcnt(kVmcnt4);
    asm volatile("s_barrier" ::: "memory");
    float s_cur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s_cur[i] = sa_nxt[i] * sb_nxt;
    // uniform per-step block indices (readfirstlane keeps the compiler from
    // deriving one pointer induction variable per unrolled step)
    const int k1n = __builtin_amdgcn_readfirstlane(kb + 1 < last ? kb + 1 : last);
    const int k2n = __builtin_amdgcn_readfirstlane(kb + 2 < last ? kb + 2 : last);
    const float* sa_row = p.sa + (int64_t)k1n * p.sa_stride;
    const float* sb_row = t.sbbase + (int64_t)k1n * p.sb_stride;
    const uint32_t kb1 = (uint32_t)k1n * BK, kb2 = (uint32_t)k2n * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o = (uint32_t)t.sa_idx[i] * 4u;
      asm volatile("" : "+v"(o));
      sa_nxt[i] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sa_row) + o);
    }
    sb_nxt = sb_row[t.nb];

    v8i af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = read_frag(a_l, wm * 64 + 16 * i, off0, off1);
    v8i bf[2];
    bf[0] = read_frag(b_l, wn * 128, off0, off1);
    v4f part[2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < 32; ++tt) {
      const int j = tt >> 2, i = tt & 3;
      part[tt & 1] =
          __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j & 1], af[i], zero, 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if ((tt & 3) == 1) {
        const int q = tt >> 2;  // A_{k+1} parts 0..3, then B_{k+2} parts 0..3
        if (q < 4)
          t.lda.issue_at(p.a, kb1, wa, wave, q);
        else
          t.ldb.issue_at(t.bbase, kb2, wb, wave, q - 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 0 && j < 7) {
        bf[(j + 1) & 1] = read_frag(b_l, wn * 128 + 16 * (j + 1), off0, off1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (tt > 0) {
        const int tp = tt - 1, jp = tp >> 2, ip = tp & 3;
        acc[ip][jp] += part[tp & 1] * s_cur[ip];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    acc[3][7] += part[1] * s_cur[3];
  };

  // A_k sits in slot 2(k-k0)+1 mod 5 and B_k in 2(k-k0) mod 5; step k fills
  // the two slots step k-1 read with A_{k+1} and B_{k+2}.  The pattern
  // repeats every five steps
  int kb = k0;
  for (; kb + 5 <= k1; kb += 5) {
    step(R.r1, R.r0, R.r3, R.r4, kb);
    step(R.r3, R.r2, R.r0, R.r1, kb + 1);
    step(R.r0, R.r4, R.r2, R.r3, kb + 2);
    step(R.r2, R.r1, R.r4, R.r0, kb + 3);
    step(R.r4, R.r3, R.r1, R.r2, kb + 4);
  }
  if (kb < k1) step(R.r1, R.r0, R.r3, R.r4, kb);
  if (kb + 1 < k1) step(R.r3, R.r2, R.r0, R.r1, kb + 1);
  if (kb + 2 < k1) step(R.r0, R.r4, R.r2, R.r3, kb + 2);
  if (kb + 3 < k1) step(R.r2, R.r1, R.r4, R.r0, kb + 3);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int A_BLK, bool GROUPED>
__global__ void __launch_bounds__(512)
gemm_ring_kernel(TiledArgs p) {
  constexpr int HALF = 256 * BK;
  __shared__ __attribute__((aligned(1024))) uint8_t r0[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r2[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r3[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r4[HALF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = wave % 4;
  const int wn = wave / 4;

  int tm, tn;
  map_tile(p, GROUPED, tm, tn);
  const int n0 = tn * BN;
  int m0 = tm * 256;
  int rows_end = p.M;
  RingTile t;
  t.bbase = p.b;
  t.sbbase = p.sb;
  const uint32_t* sfbbase = p.sfb;  // (unused: no UE8M0 form)
  if (GROUPED) {
    if (!grouped_tile(p, tm, n0, lane, m0, rows_end, t.bbase, t.sbbase, sfbbase)) return;
  }
  ring_tile_init<A_BLK>(p, t, m0, rows_end, n0, wave, lane);

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  ring_run(p, Ring{r0, r1, r2, r3, r4}, t, 0, p.nkb, wave, lane, acc);

  if constexpr (GROUPED) {
    grouped_store(p, acc, m0, n0 + wn * 128, wm * 64, rows_end, lane);
  } else {
    const int fr = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + 16 * i + fr;
      if (m >= rows_end) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = n0 + wn * 128 + 16 * j + 4 * (lane >> 4);
        if (n < p.N) {
          const float tt[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          store4<EPI_NONE, false>(p.c, m, n, tt, p.epi);  // dense ring: no epilogue
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Balanced grouped GEMM.  The grid above gives each workgroup one whole tile;
// when the tile count is a little above a multiple of the compute units
// (288 tiles for 256 CUs) the last wave leaves most of the chip idle.  Here
// one persistent workgroup per CU takes an equal share of the (tile, K
// block) work instead: whole tiles for all but the last one or two waves of
// tiles, then equal contiguous runs of K blocks over the rest, so a tile may
// be split between consecutive workgroups at any K block.  That pays while
// the matrix cores bound the launch; where streaming the weights does (the
// MoE projections), the pieces' extra traffic makes it slower.
//
// Every piece of a split tile is summed from zero in K order like a whole
// tile; each piece's FP32 accumulators go to the workspace, and the last
// workgroup to finish a piece of the tile (an arrival counter decides) adds
// the pieces in K order -- fixed by the split, not by arrival, so the result
// is deterministic -- and writes the tile through the grouped epilogue.  No
// workgroup ever waits for another.
//
// Work positions: row tiles in order of their first block, 256-column tiles
// along N inside each, tile id = row tile * tiles_n + column tile; a unit is
// one K block of one tile.

// Row tiles of the grouped layout, found by one wave walking the blocks' first
// rows 64 at a time (all lanes end with the same values).  A block starts a
// row tile when its id is a valid expert and it lies an even number of blocks
// after the first block of its run of equal ids: the pairing of grouped_tile.
// pad(b, q) is called (wave-uniformly) for every whole padding block b, q its
// rank among them.  With find >= 0 the walk stops at row tile `find` and
// returns its first block; otherwise it returns -1 and *count holds the
// number of row tiles.
template <class PadFn>
__device__ __forceinline__ int scan_row_tiles(const TiledArgs& p, int lane, int find, int* count,
                                              PadFn&& pad) {
  const int nblk = p.M / 128;
  int tiles = 0, npad = 0;
  int prev_id = INT_MIN;  // id of the block before the round (none before block 0)
  int run_start = 0;      // first block of that block's run
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int base = 0; base < nblk; base += 64) {
    const int b = base + lane;
    const bool in = b < nblk;
    const int id = in ? p.m_indices[(int64_t)b * 128] : INT_MIN;
    int up = __shfl_up(id, 1);
    if (lane == 0) up = prev_id;
    const unsigned long long starts = __ballot(in && id != up);
    const unsigned long long upto = starts & (below | (1ull << lane));
    const int s = upto ? base + 63 - __clzll((long long)upto) : run_start;
    const bool valid = in && id >= 0 && id < p.num_groups;
    const bool head = valid && ((b - s) & 1) == 0;
    const unsigned long long hmask = __ballot(head);
    unsigned long long pmask = __ballot(in && !valid);
    for (int q = npad; pmask; ++q) {
      const int bit = __ffsll((long long)pmask) - 1;
      pmask &= pmask - 1;
      pad(base + bit, q);
    }
    npad += __popcll(__ballot(in && !valid));
    if (find >= 0) {
      const int c = __popcll(hmask);
      if (find < tiles + c) {
        const unsigned long long hit = __ballot(head && __popcll(hmask & below) == find - tiles);
        return base + __ffsll((long long)hit) - 1;
      }
    }
    tiles += __popcll(hmask);
    prev_id = __shfl(id, 63);
    run_start = __shfl(s, 63);
  }
  if (count) *count = tiles;
  return -1;
}

// Tile `tile` of the balanced order: its rows, columns and the expert's
// operands.  False if it does not exist (only for inconsistent indices).
template <int A_BLK>
__device__ __forceinline__ bool balanced_tile(const TiledArgs& p, int tile, int wave, int lane,
                                              RingTile& t, int& m0, int& rows_end, int& n0) {
  const int rt = tile / p.tiles_n;
  n0 = (tile - rt * p.tiles_n) * BN;
  const int blk = scan_row_tiles(p, lane, rt, nullptr, [](int, int) {});
  if (blk < 0) return false;
  m0 = blk * 128;
  const int g = p.m_indices[m0];
  const int nblk = p.M / 128;
  const bool pair = blk + 1 < nblk && p.m_indices[(int64_t)(blk + 1) * 128] == g;
  rows_end = m0 + (pair ? 256 : 128);
  t.bbase = p.b + (int64_t)g * p.N * p.K;
  t.sbbase = p.sb + (int64_t)g * p.nkb * p.sb_stride;
  ring_tile_init<A_BLK>(p, t, m0, rows_end, n0, wave, lane);
  return true;
}

// Partial tile in the workspace: the accumulators in register order, lane l
// of wave w holding sub-tile s (= 8i + j) at float4 index (32w + s) * 64 + l,
// so that every store and load instruction of a wave covers 1 KB.  Stored and
// loaded with device-coherent cache policy (sc1: the XCDs' L2s are not
// coherent with each other), as the device-scope relaxed atomics of the
// small-M split-K do.
constexpr int kPartFloats = 256 * 256;
constexpr int kCachePolicySc1 = 1 << 4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* slot) {
  // raw buffer over one partial tile; accesses past it are dropped by the
  // hardware's range check
  return __builtin_amdgcn_make_buffer_rsrc(slot, 0, kPartFloats * 4, 0x00020000);
}

__device__ __forceinline__ void store_part(float* slot, const v4f (&acc)[4][8], int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = part_rsrc(slot);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int off = (((wave * 32 + i * 8 + j) * 64) + lane) * 16;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc[i][j]), r, off, 0,
                                             kCachePolicySc1);
    }
}

// Loads sub-tiles 8i .. 8i+7 (row group i) of a partial tile.
__device__ __forceinline__ void load_part_row(float* slot, int i, v4f (&v)[8], int wave, int lane) {
  const __amdgpu_buffer_rsrc_t r = part_rsrc(slot);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int off = (((wave * 32 + i * 8 + j) * 64) + lane) * 16;
    v[j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicySc1));
  }
}

template <int A_BLK>
__global__ void __launch_bounds__(512)
gemm_ring_balanced_kernel(TiledArgs p, int* counters, float* partials) {
  constexpr int HALF = 256 * BK;
  __shared__ __attribute__((aligned(1024))) uint8_t r0[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r1[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r2[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r3[HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t r4[HALF];
  const Ring R{r0, r1, r2, r3, r4};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = wave % 4, wn = wave / 4;

  // worker index: ids are dealt round-robin to the 8 XCDs; each XCD gets a
  // contiguous run of workers, hence of tiles (rows of A shared in its L2)
  const int G = (int)gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, per = G >> 3, extra = G & 7;
  const int w = xcd * per + min(xcd, extra) + (bid >> 3);

  // count the row tiles; zero this worker's share of the padding blocks'
  // tiles (padding tile z = rank * tiles_n + column tile goes to worker z % G)
  int rows_tiles = 0;
  scan_row_tiles(p, lane, -1, &rows_tiles, [&](int b, int q) {
    const int64_t z0 = (int64_t)q * p.tiles_n;
    int tn = (int)(((int64_t)w - z0 % G + G) % G);
    for (; tn < p.tiles_n; tn += G) zero_block(p, b * 128, tn * BN);
  });
  const int T = rows_tiles * p.tiles_n;
  const int D = T >= 2 * G ? T / G - 1 : 0;  // waves of whole tiles
  const int T_s = T - D * G;                  // tiles shared out by K block
  const int nk = p.nkb;
  const int U = T_s * nk;
  // at least a third of a tile per worker (at most about four pieces per
  // tile, so the last piece's reads stay short), and at least 4 K blocks
  const int u_min = max(4, (nk + 2) / 3);
  const int Gs = min(G, max(1, U / u_min));

  v4f acc[4][8];
  RingTile t;
  int m0, rows_end, n0;
  int* flag = reinterpret_cast<int*>(r4);  // LDS word for the arrival verdict

  // Worker v owns the units [v U / Gs, (v+1) U / Gs) of the shared tiles;
  // unit u belongs to worker ((u+1) Gs - 1) / U.  (32-bit: the host keeps
  // U * G below 2^31.)
  auto first_unit = [&](int v) { return v * U / Gs; };
  auto owner = [&](int u) { return ((u + 1) * Gs - 1) / U; };
  const int u1 = w < Gs ? first_unit(w + 1) : 0;
  int u = w < Gs ? first_unit(w) : 0;
  // Pieces: D whole tiles d G + w, then this worker's run of shared units.
  for (int d = 0;;) {
    int tile, ts = -1, k0 = 0, k1 = nk;
    if (d < D) {
      tile = d * G + w;
      ++d;
    } else if (u < u1) {
      ts = u / nk;
      k0 = u - ts * nk;
      k1 = min(nk, k0 + (u1 - u));
      u += k1 - k0;
      tile = D * G + ts;
    } else {
      break;
    }
    if (!balanced_tile<A_BLK>(p, tile, wave, lane, t, m0, rows_end, n0)) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    ring_run(p, R, t, k0, k1, wave, lane, acc);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with the ring before it is refilled
    if (k1 - k0 < nk) {
      // A piece of a split tile.  Worker v keeps its piece of tile ts in slot
      // 2v + 1 when ts is the last tile of a run that began in an earlier
      // tile, else in slot 2v (a worker's other tiles are whole).  The first
      // contributor wa is the only one whose run can begin before ts.
      const int wa = owner(ts * nk), wb = owner((ts + 1) * nk - 1);
      const int wa_slot = 2 * wa + (first_unit(wa) < ts * nk ? 1 : 0);
      auto slot = [&](int v) {
        return partials + (int64_t)(v == wa ? wa_slot : 2 * v) * kPartFloats;
      };
      // The first contributor's piece (the head of the tile, the end of its
      // run) is usually the last to finish: when the counter shows every
      // other piece already published, it neither stores its own nor counts
      // itself in.
      bool stored = true;
      if (w == wa) {
        if (threadIdx.x == 0)
          *flag = __hip_atomic_load(&counters[ts], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  wb - wa;
        __syncthreads();
        stored = *flag == 0;
        __syncthreads();  // (flag is rewritten below)
      }
      if (stored) {
        store_part(slot(w), acc, wave, lane);
        // every store of this wave has completed (is device-visible) ...
        __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
        __syncthreads();  // ... and so have those of every wave
        if (threadIdx.x == 0) {
          const int prev = __hip_atomic_fetch_add(&counters[ts], 1, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
          *flag = prev == wb - wa;
        }
        __syncthreads();
        // (the next ring run writes r4 only after its first barrier, which
        // every wave reaches after this read)
        if (*flag == 0) continue;
      }
      if (threadIdx.x == 0)  // leave the counter zeroed for the next call
        __hip_atomic_store(&counters[ts], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The last to finish adds the pieces in K order, ((P_wa + P_wa+1) + ...)
      // + P_wb, two row groups per round: the first from acc when it is this
      // worker's own, the others (this worker's too) read back from the
      // workspace.
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        v4f x[2][8];
        if (w != wa) {
          load_part_row(slot(wa), i, x[0], wave, lane);
          load_part_row(slot(wa), i + 1, x[1], wave, lane);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i + h][j] = x[h][j];
        }
        for (int c = wa + 1; c <= wb; ++c) {
          load_part_row(slot(c), i, x[0], wave, lane);
          load_part_row(slot(c), i + 1, x[1], wave, lane);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i + h][j] += x[h][j];
        }
      }
    }
    grouped_store(p, acc, m0, n0 + wn * 128, wm * 64, rows_end, lane);
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

// Balanced grouped GEMM: one workgroup per compute unit (the ring kernel
// holds all 160 KB of a CU's LDS), at most kBalancedMaxWorkers.  Used for
// up to 512 row blocks and 8 waves of possible tiles, so that the per-tile
// walks over the block ids stay short, and K up to 2^20, so that the unit
// arithmetic fits 32 bits (units * workers < 2 * 256 * 8192 * 256 = 2^30);
// larger problems keep the one-tile-per-workgroup grid, whose last wave is
// a small part of the launch.
constexpr int kBalancedMaxWorkers = 256;

namespace {

int balanced_workers() {
  static const int v = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = kBalancedMaxWorkers;
    return cus < 1 ? 1 : (cus > kBalancedMaxWorkers ? kBalancedMaxWorkers : cus);
  }();
  return v;
}

// Partial-tile slots the kernel may use with G workers: two per worker that
// takes part in the split (see gemm_ring_balanced_kernel), bounded through
// the largest possible number of split tiles.
int64_t balanced_slots(int64_t M, int64_t N, int64_t K, int64_t G) {
  const int64_t tiles = (M / 128) * ((N + BN - 1) / BN), nk = K / BK;
  const int64_t ts = tiles < 2 * G - 1 ? tiles : 2 * G - 1;
  const int64_t u_min = (nk + 2) / 3 > 4 ? (nk + 2) / 3 : 4;
  int64_t gs = ts * nk / u_min;
  gs = gs < 1 ? 1 : (gs > G ? G : gs);
  return 2 * gs;
}

}  // namespace

bool grouped_balanced_applies(int64_t M, int64_t N, int64_t K) {
  const int64_t nblk = M / 128, tiles = nblk * ((N + BN - 1) / BN);
  return nblk <= 512 && tiles <= 8 * (int64_t)kBalancedMaxWorkers && K / BK <= 8192;
}

size_t grouped_balanced_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!grouped_balanced_applies(M, N, K)) return 0;
  return kSplitkCounterBytes +
         (size_t)balanced_slots(M, N, K, kBalancedMaxWorkers) * kPartFloats * sizeof(float);
}

hipError_t launch_gemm_grouped_balanced(const GemmProblem& q, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  const int G = balanced_workers();
  const size_t need = kSplitkCounterBytes +
                      (size_t)balanced_slots(q.M, q.N, q.K, G) * kPartFloats * sizeof(float);
  if (!workspace || !grouped_balanced_applies(q.M, q.N, q.K) || workspace_bytes < need)
    return launch_gemm_tiled(q, true, stream);
  TiledArgs p;
  p.c = q.c; p.a = q.a; p.b = q.b; p.sa = q.sa; p.sb = q.sb;
  p.sfa = nullptr; p.sfb = nullptr;
  p.epi = resolved_epilogue(q);
  p.m_indices = q.m_indices; p.num_groups = q.num_groups;
  p.k_offsets = nullptr;
  p.M = (int)q.M; p.N = (int)q.N; p.K = (int)q.K;
  p.nkb = (int)(q.K / BK);
  p.sa_stride = (int)((q.M + q.a_block_rows - 1) / q.a_block_rows);
  p.sb_stride = (int)((q.N + 127) / 128);
  p.tiles_m = (int)(q.M / 128);
  p.tiles_n = (int)((q.N + BN - 1) / BN);
  p.group_m = group_m();
  p.grouped_n_major = 0;
  int* counters = static_cast<int*>(workspace);
  float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSplitkCounterBytes);
  if (q.a_block_rows == 1)
    hipLaunchKernelGGL((gemm_ring_balanced_kernel<1>), dim3(G), dim3(512), 0, stream, p, counters,
                       partials);
  else
    hipLaunchKernelGGL((gemm_ring_balanced_kernel<128>), dim3(G), dim3(512), 0, stream, p,
                       counters, partials);
  return hipGetLastError();
}

}  // namespace dg
