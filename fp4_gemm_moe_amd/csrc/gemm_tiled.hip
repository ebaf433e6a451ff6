// LDS-tiled, double-buffered scaled-MFMA GEMM for the MX modes (MXFP8 and
// MXFP4) -- the large-M tier of the flashrt/fp4-gemm page's M-tiered dispatch
// and the grouped MoE GEMMs of the HALOps "GEMM" page (group_contiguous_gemm,
// group_masked_gemm, batch_gemm sections).
//
// Structure (gfx950):
//   * 256 threads = 4 waves (one per SIMD) in a 2 x 2 grid; a block tile is
//     256 x 256 outputs, a wave tile 128 x 128 built from 4 x 4 fragments of
//     V_MFMA_SCALE_F32_32X32X64_F8F6F4 (weights as src0, activations as src1,
//     FP32 accumulation in 256 accumulation registers, E8M0 scales per 32
//     elements).  A 128 x 128 wave tile keeps the LDS fragment traffic at
//     1/128 byte per FLOP, which the LDS can serve at the matrix-core rate.
//   * A stage holds 128 bytes of every row of the A and B tiles: 128 FP8
//     elements (two MFMA steps of 64) or 256 FP4 elements (four steps).  In
//     both formats a lane reads 16-byte chunks h, 2+h, 4+h, 6+h of its
//     fragment row (h = lane / 32): FP8 pairs them as (h, 2+h), (4+h, 6+h);
//     FP4 uses each chunk as one step.
//   * Global -> LDS with 16-byte direct-to-LDS loads into an XOR-swizzled
//     layout; a wave's load fills 1 KB = 8 rows, lane j fetching the chunk
//     that belongs at slot j.
//   * Two LDS stages: the loads of step k+1 fly during step k, and the loads
//     of the first step of the workgroup's next tile fly during the last step
//     of the current tile, ahead of its epilogue stores.  Vector-memory
//     operations retire in issue order, so every wait names how many later
//     operations may stay in flight and the stores drain under the next
//     tile's first step.
//   * Persistent grid, one workgroup per compute unit.  Tiles are ordered so
//     that the 32 consecutive tiles one XCD (one L2) runs side by side cover
//     4 row tiles x 8 column tiles.
// Requirements (checked by the dispatcher): K % 128 == 0 (FP8) or
// K % 256 == 0 (FP4); scale pointers 4-byte aligned; lda * 256 < 2^31;
// n * 512 < 2^31.
#include "gemm_common.hpp"

namespace hq {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) const void* lds_cptr_t;

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row; conflict
// free for the fragment reads below (32 rows x one chunk per half wave),
// measured with the LDS bank-conflict counter.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_cptr_t)p;
}

// A pointer the compiler cannot prove uniform (it came through LDS), made
// uniform explicitly; the value is the same in every lane.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  uint64_t v = (uint64_t)(uintptr_t)p;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Direct-to-LDS loads: every lane fetches `size` bytes from sbase + voff and
// the wave's 64 results land contiguously at LDS address m0 (lane j at
// m0 + j * size).  Issued as inline assembly so that the compiler inserts no
// alias waits of its own: the kernel orders these writes explicitly (a wait
// on the vector-memory counter, then a workgroup barrier, before a stage is
// read; a barrier after the last read of a stage before it is refilled).  m0
// is set inside each statement; nothing else in the kernel uses it.
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds) : "memory");
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint32_t lds_read4(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

template <int FMT>
__device__ __forceinline__ v16f mfma32(v8i w, v8i x, v16f acc, int sw, int sx) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, x, acc, FMT, FMT, 0, sw, 0, sx);
}

constexpr int BM = 256, BN = 256;
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int WT = 128;                     // wave tile (square)
constexpr int SROW = 128;                   // bytes of a row per stage
constexpr int LOADS = BM * (SROW / 16) / THREADS;   // 16-byte loads per operand per thread (8)
constexpr int kStores = 32;                 // output stores per thread per tile

template <int FMT>
struct Cfg {
  static constexpr int SB = FMT == 0 ? 4 : 8;       // scale bytes per row per stage
  static constexpr int PLANES = SB / 4;
  static constexpr int A_BYTES = BM * SROW;
  static constexpr int B_BYTES = BN * SROW;
  static constexpr int STAGE = A_BYTES + B_BYTES + (BM + BN) * SB;
  static constexpr int OPS = 2 * LOADS + 2 * PLANES;  // vector-memory ops per stage per thread
};

// Where a tile sits: group, first row, row end and first column.
struct TileGeom {
  int g;
  int64_t row0, row_end, n0;
};

__device__ __forceinline__ TileGeom tile_geom(const GemmArgs& p, const TileTable& tt, int total_gm,
                                              int NT, int mt_per, int t) {
  // blocks of 4 m-tiles x all n-tiles, walked n-major inside the block so 32
  // consecutive tiles = 4 m x 8 n
  const int blk = t / (4 * NT);
  const int rem = t - blk * 4 * NT;
  const int mrem = total_gm - blk * 4;
  const int mb = mrem < 4 ? mrem : 4;
  const int nt = rem / mb;
  const int gm = blk * 4 + (rem - nt * mb);
  TileGeom tg;
  if (p.form == kUniform) {
    tg.g = gm / mt_per;
    int mt = gm - tg.g * mt_per;
    int64_t gs = (int64_t)tg.g * p.slot_rows;
    tg.row0 = gs + (int64_t)mt * BM;
    tg.row_end = tg.row0 + BM < gs + p.slot_rows ? tg.row0 + BM : gs + p.slot_rows;
  } else {
    tg.g = tile_group(tt, p.num_groups, gm);
    int mt = gm - (tg.g > 0 ? tt.mt_prefix[tg.g - 1] : 0);
    tg.row0 = (int64_t)tt.start[tg.g] + (int64_t)mt * BM;
    int64_t ge = (int64_t)tt.start[tg.g] + tt.count[tg.g];
    tg.row_end = tg.row0 + BM < ge ? tg.row0 + BM : ge;
  }
  tg.n0 = (int64_t)nt * BN;
  return tg;
}

// Per-thread load plan of one tile: uniform bases and per-lane offsets.
struct LoadPlan {
  const uint8_t *a_base, *b_base, *sa_base, *sb_base;
  uint32_t a_off[LOADS], b_off[LOADS];
  uint32_t sa_off, sb_off;
};

__device__ __forceinline__ LoadPlan make_plan(const GemmArgs& p, const TileGeom& tg, int w, int lane) {
  LoadPlan lp;
  lp.a_base = uniform_ptr(p.a + tg.row0 * p.lda);
  lp.b_base = uniform_ptr(p.b + (int64_t)tg.g * p.b_stride + tg.n0 * p.lda);
  lp.sa_base = uniform_ptr(p.sfa + tg.row0 * p.ldsf);
  lp.sb_base = uniform_ptr(p.sfb + (int64_t)tg.g * p.sfb_stride + tg.n0 * p.ldsf);
  const int a_rows = (int)(tg.row_end - tg.row0);
  const int b_rows = (int)(p.n - tg.n0 < BN ? p.n - tg.n0 : BN);
  // load i of wave w fills LDS rows [(i*4 + w) * 8, +8); lane j -> row + j/8,
  // physical chunk j % 8, logical chunk (j % 8) ^ swz(row).  Rows past the
  // tile end re-read a valid row (their results are never stored).
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    int row = (i * WAVES + w) * 8 + (lane >> 3);
    int c = (lane & 7) ^ swz(row);
    int ra = row < a_rows ? row : a_rows - 1;
    int rb = row < b_rows ? row : b_rows - 1;
    lp.a_off[i] = (uint32_t)(ra * p.lda + c * 16);
    lp.b_off[i] = (uint32_t)(rb * p.lda + c * 16);
  }
  // scales: wave w loads rows [64w, 64w + 64) of A and of B
  int row = w * 64 + lane;
  int ra = row < a_rows ? row : a_rows - 1;
  int rb = row < b_rows ? row : b_rows - 1;
  lp.sa_off = (uint32_t)(ra * p.ldsf);
  lp.sb_off = (uint32_t)(rb * p.ldsf);
  return lp;
}

// Issues K step k of a tile into LDS stage `st`: Cfg<FMT>::OPS operations.
template <int FMT>
__device__ __forceinline__ void issue(const LoadPlan& lp, int k, const uint8_t* st, int w) {
  using C = Cfg<FMT>;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(st));
  const uint32_t la = base + w * 1024;
  const uint32_t lb = la + C::A_BYTES;
  const uint8_t* ak = lp.a_base + k * SROW;
  const uint8_t* bk = lp.b_base + k * SROW;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) dma16(ak, lp.a_off[i], la + i * WAVES * 1024);
#pragma unroll
  for (int i = 0; i < LOADS; ++i) dma16(bk, lp.b_off[i], lb + i * WAVES * 1024);
  // scale planes: dword plane h of row r at plane h * rows + r
  const uint32_t lsa = base + C::A_BYTES + C::B_BYTES + w * 256;
  const uint32_t lsb = lsa + BM * C::SB;
#pragma unroll
  for (int h = 0; h < C::PLANES; ++h) {
    dma4(lp.sa_base + k * C::SB + 4 * h, lp.sa_off, lsa + h * BM * 4);
    dma4(lp.sb_base + k * C::SB + 4 * h, lp.sb_off, lsb + h * BN * 4);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence: the kernel's own waits order the
// LDS traffic (all fragment reads are consumed by matrix instructions before
// a wave reaches the barrier), and a fence would also wait for the epilogue
// stores.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

template <int FMT>
__global__ __launch_bounds__(THREADS, 1) void mx_gemm_tiled(GemmArgs p) {
  using C = Cfg<FMT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileTable tt;

  const int G0 = p.num_groups;
  const int NT = (int)((p.n + BN - 1) / BN);
  const int mt_per = p.form == kUniform ? (int)((p.slot_rows + BM - 1) / BM) : 0;
  int total_gm;
  if (p.form == kUniform) total_gm = G0 * mt_per;
  else total_gm = build_tile_table(p, BM, tt);
  const int total = total_gm * NT;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int lane = tid & 63;
  const int wm = w >> 1, wn = w & 1;                        // 2 x 2 wave grid
  const int h = lane >> 5, r32 = lane & 31;
  const int nk = (int)(p.lda / SROW);

  // XCD-aware order: workgroup b runs on XCD b % 8; inside a round of
  // gridDim tiles XCD x owns a contiguous run of tiles.
  const int nxcd = gridDim.x >= 8 ? 8 : 1;
  const int per_xcd = gridDim.x / nxcd;
  const int slot = (blockIdx.x % nxcd) * per_xcd + blockIdx.x / nxcd;
  const int stride = per_xcd * nxcd;
  if ((int)blockIdx.x >= stride) return;
  int t = slot;
  if (t >= total) return;

  TileGeom tg = tile_geom(p, tt, total_gm, NT, mt_per, t);
  LoadPlan lp = make_plan(p, tg, w, lane);
  int stage = 0;
  issue<FMT>(lp, 0, smem, w);
  wait_vm<0>();
  bar();

  v16f acc[4][4];

  // one K step on stage `cur`: read fragments of a half step, multiply, twice
  auto step = [&](const uint8_t* cur) {
    const uint8_t* la = cur;
    const uint8_t* lb = cur + C::A_BYTES;
    const uint8_t* lsa = cur + C::A_BYTES + C::B_BYTES;
    const uint8_t* lsb = lsa + BM * C::SB;
    uint32_t asc[4][C::PLANES], bsc[4][C::PLANES];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * WT + i * 32 + r32, rb = wn * WT + i * 32 + r32;
#pragma unroll
      for (int q = 0; q < C::PLANES; ++q) {
        asc[i][q] = lds_read4(lsa + q * BM * 4 + ra * 4);
        bsc[i][q] = lds_read4(lsb + q * BN * 4 + rb * 4);
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // chunks 4*half + h and 4*half + 2 + h of every fragment row
      uint4 a0[4], a1[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wm * WT + i * 32 + r32, rb = wn * WT + i * 32 + r32;
        const int sa = swz(ra), sb = swz(rb);
        a0[i] = lds_read16(la + ra * SROW + (((4 * half + h) ^ sa) << 4));
        a1[i] = lds_read16(la + ra * SROW + (((4 * half + 2 + h) ^ sa) << 4));
        b0[i] = lds_read16(lb + rb * SROW + (((4 * half + h) ^ sb) << 4));
        b1[i] = lds_read16(lb + rb * SROW + (((4 * half + 2 + h) ^ sb) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (FMT == 0) {
            // FP8 step `half` covers blocks 2*half + {0,1}: lane group h
            // carries block 2*half + h (byte of the single plane)
            const int sh = 8 * (2 * half + h);
            v8i af = v8i{(int)a0[i].x, (int)a0[i].y, (int)a0[i].z, (int)a0[i].w,
                         (int)a1[i].x, (int)a1[i].y, (int)a1[i].z, (int)a1[i].w};
            v8i bf = v8i{(int)b0[j].x, (int)b0[j].y, (int)b0[j].z, (int)b0[j].w,
                         (int)b1[j].x, (int)b1[j].y, (int)b1[j].z, (int)b1[j].w};
            acc[i][j] = mfma32<0>(bf, af, acc[i][j], (int)((bsc[j][0] >> sh) & 0xFFu),
                                  (int)((asc[i][0] >> sh) & 0xFFu));
          } else {
            // FP4 steps 2*half (chunk 4*half + h) and 2*half + 1 (chunk
            // 4*half + 2 + h); step v, lane group h: block 2v + h =
            // plane v/2 = half, byte 2(v%2) + h
            const int sh0 = 8 * h, sh1 = 8 * (2 + h);
            v8i af0 = v8i{(int)a0[i].x, (int)a0[i].y, (int)a0[i].z, (int)a0[i].w, 0, 0, 0, 0};
            v8i af1 = v8i{(int)a1[i].x, (int)a1[i].y, (int)a1[i].z, (int)a1[i].w, 0, 0, 0, 0};
            v8i bf0 = v8i{(int)b0[j].x, (int)b0[j].y, (int)b0[j].z, (int)b0[j].w, 0, 0, 0, 0};
            v8i bf1 = v8i{(int)b1[j].x, (int)b1[j].y, (int)b1[j].z, (int)b1[j].w, 0, 0, 0, 0};
            const uint32_t bs = bsc[j][C::PLANES - 1 - (1 - half) * (C::PLANES - 1)];
            const uint32_t as = asc[i][C::PLANES - 1 - (1 - half) * (C::PLANES - 1)];
            acc[i][j] = mfma32<4>(bf0, af0, acc[i][j], (int)((bs >> sh0) & 0xFFu), (int)((as >> sh0) & 0xFFu));
            acc[i][j] = mfma32<4>(bf1, af1, acc[i][j], (int)((bs >> sh1) & 0xFFu), (int)((as >> sh1) & 0xFFu));
          }
        }
      }
    }
  };

  bool prior_stores = false;
  while (true) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // step 0: its stage is visible.  The prefetch of step 1 is issued after
    // the previous tile's stores, so waiting for it also drains them.
    for (int k = 0; k + 1 < nk; ++k) {
      issue<FMT>(lp, k + 1, smem + (stage ^ 1) * C::STAGE, w);
      step(smem + stage * C::STAGE);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<0>();
      bar();
      stage ^= 1;
    }
    // last step: prefetch the next tile's first step
    const int t_next = t + stride;
    const bool has_next = t_next < total;
    TileGeom tg_next = tg;
    LoadPlan lp_next = lp;
    if (has_next) {
      tg_next = tile_geom(p, tt, total_gm, NT, mt_per, t_next);
      lp_next = make_plan(p, tg_next, w, lane);
      issue<FMT>(lp_next, 0, smem + (stage ^ 1) * C::STAGE, w);
    }
    step(smem + stage * C::STAGE);
    bar();                 // stage `stage` free; the next tile's step 0 is in flight
    stage ^= 1;

    // ---- epilogue: BF16 (+bias), 16-byte buffer stores relative to the
    // tile's first row.  32x32 result: lane l holds D[8b + 4(l/32) + r][l%32]
    // in register 4b + r, i.e. out[m = l%32][n = 8b + 4(l/32) + r].  Lanes l
    // and l^32 swap one 4-column quad so each lane owns 8 consecutive
    // columns: lane group 0 stores columns 8b..8b+7 for b = 0, 2 and lane
    // group 1 for b = 1, 3.
    const uint8_t* obase = uniform_ptr(reinterpret_cast<const uint8_t*>(p.out + tg.row0 * p.n));
    const uint32_t obytes = __builtin_amdgcn_readfirstlane((uint32_t)((tg.row_end - tg.row0) * p.n * 2));
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(obase), (short)0, (int)obytes, 0x00020000);
    const uint16_t* bias = p.bias ? p.bias + (int64_t)tg.g * p.n : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4f bq[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t n = tg.n0 + wn * WT + j * 32 + 8 * b + 4 * h;
        bq[b] = v4f{0.f, 0.f, 0.f, 0.f};
        if (bias != nullptr && n < p.n) {
          uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
          bq[b] = v4f{bf16_lo(bb.x), bf16_hi(bb.x), bf16_lo(bb.y), bf16_hi(bb.y)};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t mr = wm * WT + i * 32 + r32;             // row within the tile
        uint32_t pk[4][2];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          pk[b][0] = pack_bf16x2(acc[i][j][4 * b] + bq[b][0], acc[i][j][4 * b + 1] + bq[b][1]);
          pk[b][1] = pack_bf16x2(acc[i][j][4 * b + 2] + bq[b][2], acc[i][j][4 * b + 3] + bq[b][3]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {            // e = 0: quads b = 0/1, e = 1: b = 2/3
          const int bl = 2 * e, bh = 2 * e + 1;
          // group 0 sends its b = 2e+1 quad and receives the partner's b = 2e
          // quad; group 1 the other way round
          uint32_t s0 = h == 0 ? pk[bh][0] : pk[bl][0];
          uint32_t s1 = h == 0 ? pk[bh][1] : pk[bl][1];
          uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32, 64);
          uint32_t r1 = (uint32_t)__shfl_xor((int)s1, 32, 64);
          typedef uint32_t v4u __attribute__((ext_vector_type(4)));
          v4u o = h == 0 ? v4u{pk[bl][0], pk[bl][1], r0, r1} : v4u{r0, r1, pk[bh][0], pk[bh][1]};
          const int64_t n = tg.n0 + wn * WT + j * 32 + 8 * (h == 0 ? bl : bh);
          const uint32_t off = n < p.n ? (uint32_t)((mr * p.n + n) * 2) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(o, orsrc, (int)off, 0, 0);
        }
      }
    }
    if (!has_next) break;
    // the next tile's step 0 was issued before these kStores stores
    wait_vm<kStores>();
    bar();
    t = t_next;
    tg = tg_next;
    lp = lp_next;
    prior_stores = true;
  }
  (void)prior_stores;
}

template <int FMT>
hipError_t launch_tiled_cfg(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  using C = Cfg<FMT>;
  const int smem = 2 * C::STAGE;
  static bool attr_set = false;   // per process; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mx_gemm_tiled<FMT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t NT = (p.n + BN - 1) / BN;
  int64_t gm_upper;
  if (p.form == kContiguous) gm_upper = (p.m_rows + BM - 1) / BM + p.num_groups;
  else gm_upper = (int64_t)p.num_groups * ((p.slot_rows + BM - 1) / BM);
  const int64_t tiles = gm_upper * NT;
  int cus = dev.num_cus;
  if (p.cu_limit > 0 && p.cu_limit < cus) cus = p.cu_limit;
  int64_t grid = cus;
  if (tiles < grid) grid = tiles;
  if (grid >= 8) grid -= grid % 8;     // whole rounds over the 8 XCDs
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((mx_gemm_tiled<FMT>), dim3((unsigned)grid), dim3(THREADS), smem, s, p);
  return hipGetLastError();
}

}  // namespace

bool tiled_supported(const GemmArgs& p) {
  if (p.mode == kNVFP4) return false;
  const int64_t step = p.mode == kMXFP8 ? 128 : 256;
  if (p.k % step != 0) return false;
  if ((reinterpret_cast<uintptr_t>(p.sfa) | reinterpret_cast<uintptr_t>(p.sfb)) & 3) return false;
  if (p.lda * 256 >= (int64_t)1 << 31) return false;
  if (p.n * 256 * 2 > 0x7FFFFFFFLL) return false;   // 32-bit output offsets below the drop marker
  return true;
}

hipError_t launch_gemm_tiled(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  if (p.mode == kMXFP8) return launch_tiled_cfg<0>(s, p, dev);
  return launch_tiled_cfg<4>(s, p, dev);
}

}  // namespace hq
