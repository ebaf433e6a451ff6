// LDS-tiled, double-buffered GEMM for the MX modes (MXFP8 and MXFP4, scaled
// MFMA) and NVFP4 (exact FP16 decode, FP16 MFMA) -- the large-M tier of the flashrt/fp4-gemm page's M-tiered dispatch
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
//     elements (two MFMA sub-steps of 64) or 256 FP4 elements (four).  In
//     both formats a lane reads 16-byte chunks h, 2+h, 4+h, 6+h of its
//     fragment row (h = lane / 32): FP8 pairs them as (h, 2+h), (4+h, 6+h);
//     FP4 uses each chunk as one sub-step.
//   * Global -> LDS with 16-byte direct-to-LDS buffer loads into an
//     XOR-swizzled layout; a wave's load fills 1 KB = 8 rows, lane j fetching
//     the chunk that belongs at slot j.  The buffer descriptor of a tile ends
//     at the end of the operand's allocation, so rows past it are dropped by
//     the range check instead of being clamped; rows past a tile's own end
//     (a group's last partial tile) read neighbouring valid rows whose
//     results are never stored.  Per-lane load offsets are therefore the same
//     for every tile and K step.
//   * Two LDS stages: the loads of step k+1 fly during step k.  At a tile
//     boundary the loads of the next tile's first two steps are issued before
//     the epilogue stores, so the stores drain under the next tile's first
//     two steps.  Vector-memory operations retire in issue order; every wait
//     names how many later operations may stay in flight, which is correct
//     whenever at least that many were issued after the awaited one.
//   * Persistent grid, one workgroup per compute unit.  Tiles are ordered so
//     that the 32 consecutive tiles one XCD (one L2) runs side by side cover
//     4 row tiles x 8 column tiles.
// Requirements (checked by the dispatcher): K % 128 == 0 (FP8) or
// K % 256 == 0 (FP4), at least two K steps; scale pointers 4-byte aligned; lda * 256 < 2^31;
// n * 512 < 2^31.
#include <atomic>
#include <type_traits>

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

__device__ __forceinline__ uint32_t ufirst(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t ufirst64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  return (int64_t)(((uint64_t)ufirst((uint32_t)(u >> 32)) << 32) | ufirst((uint32_t)u));
}
// A pointer the compiler cannot prove uniform, made uniform explicitly; the
// value is the same in every lane.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  return (const uint8_t*)(uintptr_t)ufirst64((int64_t)(uintptr_t)p);
}

// Raw buffer descriptor over [base, base + bytes); `bytes` saturates at the
// 32-bit record limit (a tile never reads that far).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)n, 0x00020000);
}

// Direct-to-LDS buffer loads: every lane fetches `size` bytes at byte offset
// voff of the buffer (nothing if out of range) and the wave's 64 results land
// contiguously at LDS address m0 (lane j at m0 + j * size).  Issued as inline
// assembly so that the compiler inserts no alias waits of its own: the kernel
// orders these writes explicitly (a wait on the vector-memory counter, then a
// workgroup barrier, before a stage is read; a barrier after the last read of
// a stage before it is refilled).  m0 is set inside each statement; nothing
// else in the kernel uses it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r),
               "s"(lds) : "memory");
}
// The same with the non-temporal cache policy, for operands read exactly
// once: a microbenchmark streaming a weight tensor in a tile's row pattern
// (256 rows x 128 bytes per step, one workgroup per CU) reads 7.0 TB/s with
// it and 4.6 TB/s without.
__device__ __forceinline__ void dma16nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(r),
               "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(r),
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
constexpr int kMB = 8;                      // m-tiles per block of the tile order (make_tile)
constexpr int SROW = 128;                   // bytes of a row per stage
constexpr int kNV = 2;                      // format tag of the NVFP4 instantiation
constexpr int kSkSpin = 1 << 20;            // polls of a stream-K flag before giving up (~1 s)

template <int FMT>
struct Cfg {
  // 32x32 fragments per wave along M and N: FP8 and NVFP4 run 4 waves of
  // 128 x 128, FP4 8 waves (two per SIMD) of 128 x 64 (measured faster)
  static constexpr int FI = 4, FJ = FMT == 4 ? 2 : 4;
  static constexpr int WTM = 32 * FI, WTN = 32 * FJ;    // wave tile
  static constexpr int WGN = BN / WTN;                  // waves along N
  static constexpr int WAVES = (BM / WTM) * WGN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int LOADS = BM * (SROW / 16) / THREADS;   // 16-byte loads per operand per thread
  static constexpr int kStores = FI * FJ * 2;           // output stores per thread per tile
  // scale bytes per row per stage: 128 FP8 / 256 FP4 elements per stage in
  // E8M0 groups of 32, or 256 NVFP4 elements in UE4M3 groups of 16
  static constexpr int SB = FMT == 0 ? 4 : (FMT == 4 ? 8 : 16);
  static constexpr int PLANES = SB / 4;
  static constexpr int A_BYTES = BM * SROW;
  static constexpr int B_BYTES = BN * SROW;
  static constexpr int STAGE = A_BYTES + B_BYTES + (BM + BN) * SB;
  // vector-memory ops per stage per thread: each wave loads the scale
  // dwords of 512 / WAVES rows (of A or B with 8 waves, of both with 4)
  static constexpr int SOPS = (BM + BN) / (WAVES * 64);
};

// LDS layout and scale-load schedule.  GS (grouped scales): a row's scale
// bytes are fetched 16 at a time -- SPG consecutive K steps' worth (4 FP8,
// 2 FP4, 1 NVFP4 steps) -- by one 16-byte load per row into one of two
// scale buffers [BM + BN rows][16 bytes] next to the two operand stages.
// Each such load touches one cache line per row, so against one dword load
// per row and 4-byte plane per step this cuts the memory transactions of
// the scales 4x (the scale loads touched as many cache lines as the operand
// loads; without them the MX GEMMs ran 13-21 % faster).  It needs a row's
// scale bytes to be a multiple of 16 (K % 512 == 0 for MX); otherwise each
// stage carries its step's scales as dword planes (plane h of row r at
// h * rows + r), one dword load per row and plane.
template <int FMT, bool GS>
struct Lay {
  using C = Cfg<FMT>;
  static constexpr int STAGE = C::A_BYTES + C::B_BYTES + (GS ? 0 : (BM + BN) * C::SB);
  static constexpr int SBUF = (BM + BN) * 16;          // one scale buffer (GS)
  static constexpr int SMEM = 2 * STAGE + (GS ? 2 * SBUF : 0);
  static constexpr int SPG = GS ? 16 / C::SB : 1;      // K steps per scale load
  static constexpr int RS = GS ? 16 : 4;               // LDS bytes from row to row
  static constexpr int PS = GS ? 4 : BM * 4;           // LDS bytes from plane to plane
  static constexpr int BOFF = BM * (GS ? 16 : C::SB);  // B's scales after A's
  // vector-memory operations of a step that loads scales, and of step 1
  static constexpr int SCALE_OPS = GS ? C::SOPS : C::SOPS * C::PLANES;
  static constexpr int OPS1 = 2 * C::LOADS + (SPG == 1 ? SCALE_OPS : 0);
};

// MXFP8 load schedule (grouped scales).  A step runs its MFMA groups (i, v)
// -- fragment row i, sub-step v, four MFMAs j -- in i-major order, and issue
// slot 8 i + 4 v + j follows MFMA (i, v, j).  The next step's 16 loads per
// wave are spread over the 32 slots, one every one to three MFMAs: a burst of
// loads fills the texture-address queue and stalls the wave with no matrix
// instruction queued.  The B rows and the A rows of fragment row 0 (A loads
// i % 4 == 0) go first and are waited for at the end of the step.  The A rows
// of fragment rows 1-3 go last and are waited for in the next step, at slot
// SYNC, where the A fragment of row 1 is first read (behind a second
// workgroup barrier), so they land up to half a step later.  Measured on the
// grouped, fused and backward MXFP8 GEMMs: 4-5 % faster than all loads in the
// first half of the step, all waited for at its end.  ON = false keeps an
// instantiation on the v-major order with every load in the first half of the
// step (the row-quantising dSwiGLU epilogue, which already holds 256 VGPRs:
// the i-major loop's B fragments of both sub-steps spill there, 12 % slower).
template <int FMT, bool GS, bool ON = true>
struct Sched {
  static constexpr bool LATE = FMT == 0 && GS && ON;
  static constexpr int SLOTS = 32;              // MFMAs of a step
  static constexpr int SYNC = 4;                // slot of the mid-step wait and barrier
  static constexpr int N_LATE = 6;              // late loads per wave, the last ones issued
  static constexpr int EARLY_BEFORE_SYNC = 3;   // loads issued in slots below SYNC
  // A load i is id i, B load i id 8 + i; the late ones are A loads i % 4 != 0
  static constexpr int kSlot[16] = {0, 15, 21, 27, 3, 18, 24, 30, 1, 4, 6, 7, 9, 10, 12, 13};
  static constexpr bool late(int id) { return id < 8 && id % 4 != 0; }
  // issue slot of load `id` of `nloads` over `slots` slots
  static constexpr int slot(int id, int slots, int nloads) { return LATE ? kSlot[id] : id * slots / nloads; }
  static constexpr bool valid() {
    int n_late = 0, n_before = 0, last_early = -1, first_late = SLOTS;
    for (int id = 0; id < 16; ++id) {
      const int t = kSlot[id];
      if (t < 0 || t >= SLOTS) return false;
      for (int o = 0; o < id; ++o)
        if (kSlot[o] == t) return false;
      if (late(id)) {
        ++n_late;
        first_late = t < first_late ? t : first_late;
      } else {
        last_early = t > last_early ? t : last_early;
        if (t < SYNC) ++n_before;
      }
    }
    // every late load is issued after every early one, and none before SYNC
    return n_late == N_LATE && n_before == EARLY_BEFORE_SYNC && last_early < first_late && first_late >= SYNC;
  }
  static_assert(!LATE || (Cfg<FMT>::LOADS == 8 && Cfg<FMT>::FI == 4 && Cfg<FMT>::FJ == 4 && valid()),
                "the MXFP8 load schedule assumes 8 + 8 loads and 4 x 4 fragments per wave");
};

// Grouped forms: per group its end row and the inclusive prefixes of its
// heavy and light m-tiles.  Where two waves share each SIMD (Cfg::WAVES > 4),
// a group's last m-tile with at most WTM valid rows is light: only the waves
// of its first WTM rows multiply, at about half a heavy tile's cost.  Heavy
// m-tiles are numbered first and the grid walks its rounds in alternating
// directions, so each workgroup's share of heavy and light tiles evens out.
// With one wave per SIMD every m-tile counts as heavy.
struct TiledTable {
  int end[kMaxGroups];
  int heavy[kMaxGroups];
  int light[kMaxGroups];
};

__device__ __forceinline__ int64_t group_start(const GemmArgs& p, const TiledTable& t, int g) {
  if (p.form == kContiguous) return g > 0 ? t.end[g - 1] : 0;
  return (int64_t)g * p.slot_rows;
}

// First group whose inclusive prefix exceeds x.
__device__ __forceinline__ int prefix_group(const int* pre, int G, int x) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] > x) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Fills the table (all threads must call); returns the number of group
// m-tiles and sets n_heavy.  Device-side ends and counts are clamped as for
// every grouped form.
template <int FMT>
__device__ int build_tiled_table(const GemmArgs& p, TiledTable& t, int& n_heavy) {
  constexpr bool kSplit = Cfg<FMT>::WAVES > 4;
  constexpr int WTM = Cfg<FMT>::WTM;
  const int G = p.num_groups;
  if (p.form == kContiguous) {
    load_clamped_ends<Cfg<FMT>::THREADS>(t.end, p.group_end, G, p.m_rows);
  } else {
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
      const int64_t v = p.counts[g];
      const int64_t c = v < 0 ? 0 : (v > p.slot_rows ? p.slot_rows : v);
      t.end[g] = (int)((int64_t)g * p.slot_rows + c);
    }
    __syncthreads();
  }
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int rows = (int)(t.end[g] - group_start(p, t, g));
    const int full = rows / BM, rem = rows - full * BM;
    const bool lt = kSplit && rem > 0 && rem <= WTM;
    t.heavy[g] = full + (rem > 0 && !lt ? 1 : 0);
    t.light[g] = lt ? 1 : 0;
  }
  __syncthreads();
  n_heavy = block_scan_1024<Cfg<FMT>::THREADS>(t.heavy, G, OpAdd(), 0);
  return n_heavy + block_scan_1024<Cfg<FMT>::THREADS>(t.light, G, OpAdd(), 0);
}

// Where a tile sits (uniform): group, first row, row end, first column, and
// the byte bases / extents of its operands.
struct Tile {
  int g;
  int nk, slice;                 // K steps of this tile (range), K-split slice
  int sk0, sk1;                  // stream-K piece: K units [sk0, sk1) of the tile's units
  int sg;                        // scale buffer of the tile's first scale group (GS)
  int64_t row0, row_end, n0;
  int64_t vend;                  // end of the rows an epilogue writes (SwiGLU: the valid rows)
  const uint8_t *a, *b, *sa, *sb;
  int64_t a_bytes, b_bytes, sa_bytes, sb_bytes;
};

// `unit`: K-split slice boundaries fall on multiples of this many steps (a
// scale group with grouped scales).
// tile_cols: output columns per n-tile (BN; 128 y columns for the SwiGLU epilogue,
// whose tile spans 128 gate and 128 up weight rows).
template <int FMT>
__device__ __forceinline__ Tile make_tile(const GemmArgs& p, const TiledTable& tt, int total_gm,
                                          int n_heavy, int NT, int mt_per, int nk, int t, int unit,
                                          int tile_cols, int sk0 = 0, int sk1 = 0) {
  // K split: units are numbered slice-major, so that neighbouring units of
  // one slice share operand rows as without a split
  const int S = p.ksplit > 1 ? p.ksplit : 1;
  int slice = 0;
  if (S > 1) {
    const int per_slice = total_gm * NT;
    slice = t / per_slice;
    t -= slice * per_slice;
  }
  // blocks of 8 m-tiles x all n-tiles, walked n-major inside the block so 32
  // consecutive tiles (one XCD's share of a round) = 8 m x 4 n (measured 2 %
  // faster on the grouped MXFP8 GEMMs than blocks of 4 m-tiles)
  const int blk = t / (kMB * NT);
  const int rem = t - blk * kMB * NT;
  const int mrem = total_gm - blk * kMB;
  const int mb = mrem < kMB ? mrem : kMB;
  const int nt = rem / mb;
  const int gm = blk * kMB + (rem - nt * mb);
  int g;
  int64_t row0, row_end;
  if (p.form == kUniform) {
    g = gm / mt_per;
    const int mt = gm - g * mt_per;
    const int64_t gs = (int64_t)g * p.slot_rows;
    row0 = gs + (int64_t)mt * BM;
    row_end = row0 + BM < gs + p.slot_rows ? row0 + BM : gs + p.slot_rows;
  } else {
    int mt;
    if (gm < n_heavy) {
      g = prefix_group(tt.heavy, p.num_groups, gm);
      mt = gm - (g > 0 ? tt.heavy[g - 1] : 0);
    } else {                          // a light tile: the group's last m-tile
      g = prefix_group(tt.light, p.num_groups, gm - n_heavy);
      mt = tt.heavy[g] - (g > 0 ? tt.heavy[g - 1] : 0);
    }
    row0 = group_start(p, tt, g) + (int64_t)mt * BM;
    const int64_t ge = tt.end[g];
    row_end = row0 + BM < ge ? row0 + BM : ge;
  }
  Tile tl;
  tl.sg = 0;
  tl.g = (int)ufirst((uint32_t)g);
  // this slice's K steps [k0, k1) of the nk steps, on multiples of `unit`
  // (a stream-K piece: units [sk0, sk1) of `unit` steps)
  int k0, k1;
  if (sk1 > 0) {
    k0 = unit * sk0;
    k1 = unit * sk1;
  } else {
    const int ng = nk / unit;
    k0 = unit * (int)((int64_t)slice * ng / S);
    k1 = unit * (int)((int64_t)(slice + 1) * ng / S);
  }
  tl.sk0 = (int)ufirst((uint32_t)sk0);
  tl.sk1 = (int)ufirst((uint32_t)sk1);
  tl.slice = (int)ufirst((uint32_t)slice);
  tl.nk = (int)ufirst((uint32_t)(k1 - k0));
  const int64_t kb = (int64_t)ufirst((uint32_t)k0) * SROW, ksb = (int64_t)ufirst((uint32_t)k0) * Cfg<FMT>::SB;
  tl.row0 = ufirst64(row0);
  tl.row_end = ufirst64(row_end);
  tl.vend = tl.row_end;
  if (p.valid != nullptr) {         // the first valid[g] rows of the group (contiguous form)
    const int64_t gs = ufirst64(group_start(p, tt, tl.g));
    int64_t c = p.valid[tl.g];
    c = c < 0 ? 0 : c;
    if (gs + c < tl.vend) tl.vend = ufirst64(gs + c);
  }
  tl.n0 = (int64_t)nt * tile_cols;
  // the group's weights: one tensor of all groups, or its own allocation
  const bool discrete = p.b_ptrs != nullptr;
  const uint8_t* bbase = discrete ? reinterpret_cast<const uint8_t*>(p.b_ptrs[tl.g]) : p.b;
  const uint8_t* sbbase = discrete ? reinterpret_cast<const uint8_t*>(p.sfb_ptrs[tl.g]) : p.sfb;
  const int64_t brow0 = (discrete ? 0 : (int64_t)tl.g * p.n) + tl.n0;   // first weight row
  const int64_t brows = discrete ? p.n : (int64_t)p.num_groups * p.n;
  tl.a = uniform_ptr(p.a + tl.row0 * p.lda + kb);
  tl.b = uniform_ptr(bbase + brow0 * p.lda + kb);
  tl.sa = uniform_ptr(p.sfa + tl.row0 * p.ldsf + ksb);
  tl.sb = uniform_ptr(sbbase + brow0 * p.ldsf + ksb);
  // A rows past the tile's valid rows (the next group's, or a masked slot's
  // padding) are not fetched: the bounded loads fill them with zeros.
  // Extents count from the slice's first K byte.
  tl.a_bytes = (tl.row_end - tl.row0) * p.lda - kb;
  tl.b_bytes = (brows - brow0) * p.lda - kb;
  tl.sa_bytes = (tl.row_end - tl.row0) * p.ldsf - ksb;
  tl.sb_bytes = (brows - brow0) * p.ldsf - ksb;
  return tl;
}

// Per-lane load offsets, the same for every tile and step.  Load i of wave w
// fills LDS rows [(i*4 + w) * 8, +8) of the A and of the B tile; lane j ->
// row + j/8, physical chunk j % 8, logical chunk (j % 8) ^ swz(row).  Scale
// dwords: wave w loads rows [64w, 64w + 64).
// PAIRED (the gate|up GEMM with the SwiGLU epilogue): B-tile row r holds the
// weight row paired_row(r) past the tile's first gate row, so that fragment
// j < 2 of a wave holds gate columns and fragment j + 2 the up columns of the
// same 32 outputs: r = 128 wn + 32 j + t -> y column 64 wn + 32 (j & 1) + t,
// plus h for the up half (j >= 2).
__device__ __forceinline__ int paired_row(int r, int64_t h) {
  return 64 * (r >> 7) + 32 * ((r >> 5) & 1) + (r & 31) + ((r >> 6) & 1) * (int)h;
}

template <int FMT, bool PAIRED>
struct LoadOffsets {
  uint32_t tile[Cfg<FMT>::LOADS];
  uint32_t btile[PAIRED ? Cfg<FMT>::LOADS : 1];   // B's own offsets (PAIRED)
  uint32_t scale, bscale;
};

template <int FMT, bool PAIRED>
__device__ __forceinline__ LoadOffsets<FMT, PAIRED> make_offsets(const GemmArgs& p, int w, int lane) {
  constexpr int LOADS = Cfg<FMT>::LOADS, WAVES = Cfg<FMT>::WAVES;
  LoadOffsets<FMT, PAIRED> o;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int row = (i * WAVES + w) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    o.tile[i] = (uint32_t)(row * p.lda + c * 16);
    if constexpr (PAIRED) o.btile[i] = (uint32_t)(paired_row(row, p.h) * p.lda + c * 16);
  }
  const int srow = ((w * 64) % BM) + lane;
  o.scale = (uint32_t)(srow * p.ldsf);
  o.bscale = PAIRED ? (uint32_t)(paired_row(srow, p.h) * p.ldsf) : o.scale;
  return o;
}

// Issues K step k of tile `tl` into the LDS stage at byte address `base`
// (lds0: the LDS byte address of the dynamic LDS): 2 LOADS operand loads and
// the step's scale loads, if it has any.  part -1 issues all of them.  With
// part >= 0 only the operand loads of one of `slots` issue slots are issued
// (the 2 LOADS loads spread evenly over the slots; per-step scale planes ride
// with the last one); calls for every slot 0 .. slots-1 together issue the
// operand loads in the same order.  part -2 issues only grouped scale loads:
// the step calls it ahead of its matrix instructions, because the branch on
// the step's place in its scale group would otherwise let the compiler sink
// the instructions before it below it and bunch up the operand loads.  SCH:
// the ON flag of the instantiation's load schedule (Sched).  NTB: B's rows are
// read with the non-temporal policy (each weight byte is read once).
template <int FMT, bool GS, bool PAIRED, bool SCH = true, bool NTB = false>
__device__ __forceinline__ void issue(const Tile& tl, const LoadOffsets<FMT, PAIRED>& o, int k, uint32_t base,
                                      uint32_t lds0, int w, int part = -1, int slots = 1) {
  using C = Cfg<FMT>;
  using L = Lay<FMT, GS>;
  constexpr int LOADS = C::LOADS, WAVES = C::WAVES;
  const uint32_t la = base + w * 1024;
  const uint32_t lb = la + C::A_BYTES;
  const int64_t ka = (int64_t)k * SROW, ks = (int64_t)k * C::SB;
  const __amdgpu_buffer_rsrc_t ra = rsrc(tl.a + ka, tl.a_bytes - ka);
  const __amdgpu_buffer_rsrc_t rb = rsrc(tl.b + ka, tl.b_bytes - ka);
  if (part != -2) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (part < 0 || part == Sched<FMT, GS, SCH>::slot(i, slots, 2 * LOADS)) dma16(ra, o.tile[i], la + i * WAVES * 1024);
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      if (part < 0 || part == Sched<FMT, GS, SCH>::slot(LOADS + i, slots, 2 * LOADS)) {
        if constexpr (NTB) dma16nt(rb, PAIRED ? o.btile[i] : o.tile[i], lb + i * WAVES * 1024);
        else dma16(rb, PAIRED ? o.btile[i] : o.tile[i], lb + i * WAVES * 1024);
      }
  }
  // Scales.  With four waves wave w loads rows [64 w, 64 w + 64) of A and of
  // B; with eight, waves 0-3 those rows of A and waves 4-7 of B.
  if constexpr (GS) {
    // the first step of a scale group: the group's 16 bytes of every row
    // into scale buffer (sg + group) % 2, row r at 16 r
    if (part >= 0 || k % L::SPG != 0) return;
    const uint32_t sbuf = lds0 + 2 * L::STAGE + ((tl.sg + k / L::SPG) & 1) * L::SBUF;
    const uint32_t lsa = sbuf + ((w * 64) % BM) * 16;
    const uint32_t lsb = lsa + L::BOFF;
    const __amdgpu_buffer_rsrc_t rsa = rsrc(tl.sa + ks, tl.sa_bytes - ks);
    const __amdgpu_buffer_rsrc_t rsb = rsrc(tl.sb + ks, tl.sb_bytes - ks);
    if constexpr (C::SOPS == 2) {
      dma16(rsa, o.scale, lsa);
      dma16(rsb, o.bscale, lsb);
    } else {
      const bool is_a = w * 64 < BM;
      dma16(is_a ? rsa : rsb, is_a ? o.scale : o.bscale, is_a ? lsa : lsb);
    }
    return;
  }
  if (part == -2 || (part >= 0 && part != (2 * LOADS - 1) * slots / (2 * LOADS))) return;
  // dword plane h of row r at plane h * rows + r
  const uint32_t lsa = base + C::A_BYTES + C::B_BYTES + ((w * 64) % BM) * 4;
  const uint32_t lsb = lsa + BM * C::SB;
  const __amdgpu_buffer_rsrc_t rsa = rsrc(tl.sa + ks, tl.sa_bytes - ks);
  const __amdgpu_buffer_rsrc_t rsb = rsrc(tl.sb + ks, tl.sb_bytes - ks);
  if constexpr (C::SOPS == 2) {
#pragma unroll
    for (int h = 0; h < C::PLANES; ++h) {
      dma4(rsa, o.scale + 4 * h, lsa + h * BM * 4);
      dma4(rsb, o.bscale + 4 * h, lsb + h * BN * 4);
    }
  } else {
    const bool is_a = w * 64 < BM;
    const __amdgpu_buffer_rsrc_t rs = is_a ? rsa : rsb;
    const uint32_t ls = is_a ? lsa : lsb;
    const uint32_t so = is_a ? o.scale : o.bscale;
#pragma unroll
    for (int h = 0; h < C::PLANES; ++h) dma4(rs, so + 4 * h, ls + h * BM * 4);
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

// Two FP32 values -> packed binary16 pair (low half = a), round to nearest
// even (Inf beyond the largest finite value).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}

// Two FP32 values -> packed BF16 pair (low half = a), round to nearest even,
// in one hardware conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Epilogues (separate instantiations, so that one costs the others no
// registers): kEpiBf16 writes the BF16 output (kEpiF16: binary16, for
// p.out_f16); kEpiSplit (the launch has a
// K split, p.ksplit > 1) writes FP32 partial tiles; kEpiSwiglu (MXFP8, p.h > 0,
// PAIRED B rows) applies SwiGLU and the MXFP8 re-quant and writes codes and
// scales of y instead of the gate|up output; kEpiDswiglu (the backward
// GEMM, grouped-contiguous) applies the dSwiGLU derivative to R with the
// forward activations C and writes D and the dprob row sums; kEpiStream
// (a dense stream-K launch) runs pieces of tiles: a piece that does not end
// its tile hands its FP32 partial tile to the piece that does, which adds
// it and writes the BF16 / binary16 output.
constexpr int kEpiBf16 = 0, kEpiSplit = 1, kEpiSwiglu = 2, kEpiF16 = 3, kEpiDswiglu = 4, kEpiDswigluQ = 5,
              kEpiStream = 6;

// NOBIAS (the SwiGLU epilogue without a bias): the epilogue packs the
// accumulators as they are instead of adding a zero bias to each.  The
// result is the same: an accumulator is never -0 (the first matrix
// instruction of a tile adds its products to +0), so adding +0 changes no
// bit; the adds cost 0.7-1.5 % of the fused gate|up GEMM (interleaved A/B).
template <int FMT, int EPI, bool GS, bool NTB = false, bool NOBIAS = false>
__global__ __launch_bounds__(Cfg<FMT>::THREADS, 1) void mx_gemm_tiled(GemmArgs p) {
  using C = Cfg<FMT>;
  using L = Lay<FMT, GS>;
  constexpr int FI = C::FI, FJ = C::FJ, WTM = C::WTM, WTN = C::WTN, WGN = C::WGN;
  // vector-memory operations of the epilogue (at least; the waits below rely
  // on no fewer being issued after the next tile's loads)
  // (kEpiDswiglu issues FI * FJ * 4 stores after its loads of C; a smaller
  // count only makes the waits stricter, and vmcnt holds at most 63)
  constexpr bool DSW = EPI == kEpiDswiglu || EPI == kEpiDswigluQ;
  constexpr int kStores = EPI == kEpiSwiglu ? FI * 2 * 3 : (DSW ? 32 : C::kStores);
  static_assert(!DSW || FI * FJ * 4 >= 32, "the dSwiGLU epilogues issue at least 32 stores");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TiledTable tt;

  const int G0 = p.num_groups;
  constexpr bool PAIRED = EPI == kEpiSwiglu;
  static_assert(!PAIRED || (FMT == 0 && Cfg<FMT>::FJ == 4), "the SwiGLU epilogue pairs fragments j and j + 2");
  constexpr int TCOLS = PAIRED ? 128 : BN;                  // output columns per n-tile
  const int NT = (int)(((PAIRED ? p.h : p.n) + TCOLS - 1) / TCOLS);
  const int mt_per = p.form == kUniform ? (int)((p.slot_rows + BM - 1) / BM) : 0;
  int total_gm, n_heavy = 0;
  if (p.form == kUniform) total_gm = G0 * mt_per;
  else total_gm = build_tiled_table<FMT>(p, tt, n_heavy);
  int total = total_gm * NT * (p.ksplit > 1 ? p.ksplit : 1);
  if (p.tile_limit > 0 && p.tile_limit < total) total = p.tile_limit;   // a leading run of tiles

  const int tid = threadIdx.x;
  const int w = ufirst(tid >> 6);                           // wave index (uniform)
  const int lane = tid & 63;
  const int wm = w / WGN, wn = w % WGN;                     // wave grid (M x N)
  const int h = lane >> 5, r32 = lane & 31;
  const int nk = (int)(p.lda / SROW);          // K steps of a whole row (at least 2)

  // XCD-aware order: workgroup b runs on XCD b % 8; inside a round of
  // gridDim tiles XCD x owns a contiguous run of tiles.  Rounds alternate
  // direction: in odd rounds the workgroup at slot s takes the round's tile
  // stride - 1 - s (a workgroup's tile index still grows round by round).
  // Dense launches (one group, unsplit, the whole tile list) instead give XCD
  // x the contiguous eighth [lo_x, tile_end) of the tile list, walked 32 tiles
  // a round: its L2 then holds an eighth of the n-tiles' weights for the whole
  // launch (dense MXFP4 4096x17408x5120: 3.5 % faster, MXFP8 2 %; the grouped
  // and masked GEMMs ran 1-10 % slower with it, their groups' tiles being
  // spread over the XCDs already).
  const int nxcd = gridDim.x >= 8 ? 8 : 1;
  const int per_xcd = gridDim.x / nxcd;
  const int slot = (blockIdx.x % nxcd) * per_xcd + blockIdx.x / nxcd;
  const int stride = per_xcd * nxcd;
  if ((int)blockIdx.x >= stride) return;
  constexpr bool SKM = EPI == kEpiStream;
  const bool xmajor = !SKM && p.form == kUniform && p.num_groups == 1 && p.ksplit <= 1 && p.tile_limit <= 0;
  const int xi = (int)(blockIdx.x % nxcd), ci = (int)(blockIdx.x / nxcd);
  const int lo_x = (int)((int64_t)total * xi / nxcd);
  const int tile_end = xmajor ? (int)((int64_t)total * (xi + 1) / nxcd) : total;
  // Stream-K: workgroup b belongs to group x = b % nxcd (the XCD that the
  // round-robin dispatch gives it) at index l = b / nxcd of the group's
  // per_xcd workgroups; group x takes the tiles [total x / nxcd,
  // total (x + 1) / nxcd), whose K steps, in tile order, are units of
  // p.sk_unit steps, upt per tile, dealt out in equal runs [u0, u1) to its
  // workgroups -- at most one tile's worth each (the launcher keeps a group's
  // tiles at most its workgroups), so at most two pieces: the start of tile
  // (u1 - 1) / upt first, then the end of tile u0 / upt.  A tile's pieces
  // thus sit in one group, and the pieces before its last one in workgroups
  // of lower index: dispatched earlier, and never waiting before they hand
  // their partial on, so every wait for them ends even when the workgroups
  // are not all resident at once.  The group's tiles are neighbours in the
  // tile order (sharing B columns) and meet in one L2.  The pieces are
  // recomputed where they are needed, from an opaque copy of the workgroup
  // index, so that none of it stays in registers through the K loop.
  const int upt = SKM ? p.sk_upt : 1;
  struct Piece {
    int t, a, b;   // tile, K units [a, b) of its upt
  };
  struct SkRun {
    int64_t u0, u1;      // this workgroup's units (global numbering)
    int64_t g0, gu;      // the group's first unit and its unit count
    int base;            // slot of the group's first workgroup
  };
  auto sk_run = [&]() -> SkRun {
    int b = (int)blockIdx.x;
    asm volatile("" : "+s"(b));
    const int x = b % nxcd, l = b / nxcd;
    const int64_t t0 = (int64_t)total * x / nxcd, t1 = (int64_t)total * (x + 1) / nxcd;
    SkRun r;
    r.g0 = t0 * upt;
    r.gu = (t1 - t0) * upt;
    r.u0 = r.g0 + (int64_t)l * r.gu / per_xcd;
    r.u1 = r.g0 + (int64_t)(l + 1) * r.gu / per_xcd;
    r.base = x * per_xcd;
    return r;
  };
  auto piece = [&](int round) -> Piece {
    Piece pc{total, 0, 0};
    if constexpr (SKM) {
      const SkRun rn = sk_run();
      const int64_t u0 = rn.u0, u1 = rn.u1;
      if (u1 > u0 && u1 - u0 <= upt) {
        const int tlo = (int)(u0 / upt), thi = (int)((u1 - 1) / upt);
        if (round == 0) pc = thi > tlo ? Piece{thi, 0, (int)(u1 - (int64_t)thi * upt)}
                                       : Piece{tlo, (int)(u0 - (int64_t)tlo * upt), (int)(u1 - (int64_t)tlo * upt)};
        else if (round == 1 && thi > tlo) pc = Piece{tlo, (int)(u0 - (int64_t)tlo * upt), upt};
      }
    }
    return pc;
  };
  // the second piece, kept in LDS through the first one's K loop
  __shared__ int sk_second[3];
  Piece sk_first{total, 0, 0};
  if constexpr (SKM) {
    sk_first = piece(0);
    const Piece p1 = piece(1);
    if (tid == 0) {
      sk_second[0] = p1.t;
      sk_second[1] = p1.a;
      sk_second[2] = p1.b;
    }
  }
  auto tile_of = [&](int round) {
    if constexpr (SKM) return round == 0 ? sk_first.t : total;
    return xmajor ? lo_x + round * per_xcd + ci : round * stride + ((round & 1) ? stride - 1 - slot : slot);
  };
  const int kunit = SKM ? p.sk_unit : L::SPG;           // make_tile's K unit
  int round = 0;
  int t = tile_of(0);
  if (t >= tile_end) return;

  const LoadOffsets<FMT, PAIRED> lo = make_offsets<FMT, PAIRED>(p, w, lane);

  // Fragment-read offsets.  Fragment row i of the wave tile is LDS row
  // 128 wm + 32 i + r32 (A) / 128 wn + 32 i + r32 (B); its swizzle is
  // s0 ^ 4 (i & 1) with s0 = swz(r32), so logical chunk c + h (c even) of
  // row i sits at physical chunk ((c ^ 4 (i & 1)) | h) ^ s0.  xo[e] holds
  // the lane's byte offset of logical chunk 2e + h in an i = 0 row; row i
  // adds i * 4096 and flips e by 2 (i & 1).
  const int s0 = swz(r32);
  uint32_t xo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) xo[e] = (uint32_t)(r32 * SROW + ((((2 * e) | h) ^ s0) << 4));
  auto rd16 = [&](const uint8_t* wbase, int i, int c) -> uint4 {
    return lds_read16(wbase + i * 32 * SROW + xo[(c ^ (4 * (i & 1))) >> 1]);
  };

  v16f acc[FI][FJ];

  // One K step on stage `cur`.  A step is SUB matrix-core sub-steps (two of
  // K 64 for FP8, four of K 64 for FP4); sub-step v reads, per fragment row,
  // chunks (4v + h, 4v + 2 + h) for FP8 and chunk 2v + h for FP4.  Fragment
  // reads run one MFMA row ahead: while row i of sub-step v multiplies, the A
  // fragment of row i + 1 and the B fragment j = i of sub-step v + 1 are read,
  // so at most two B sets and two A fragments are live.  Scheduling fences
  // keep the compiler from sinking the reads onto their first use.
  constexpr int SUB = FMT == 0 ? 2 : 4;
  struct Frag {
    uint4 x, y;
  };
  auto rd = [&](const uint8_t* wbase, int i, int v) -> Frag {
    Frag f;
    if (FMT == 0) {
      f.x = rd16(wbase, i, 4 * v);
      f.y = rd16(wbase, i, 4 * v + 2);
    } else {
      f.x = rd16(wbase, i, 2 * v);
      f.y = make_uint4(0, 0, 0, 0);
    }
    return f;
  };
  auto op = [](const Frag& f) -> v8i {
    return FMT == 0 ? v8i{(int)f.x.x, (int)f.x.y, (int)f.x.z, (int)f.x.w,
                          (int)f.y.x, (int)f.y.y, (int)f.y.z, (int)f.y.w}
                    : v8i{(int)f.x.x, (int)f.x.y, (int)f.x.z, (int)f.x.w, 0, 0, 0, 0};
  };
  // scale byte of sub-step v for lane group h: FP8 block 2v + h of the one
  // dword plane; FP4 block 2v + h = plane v / 2, byte 2 (v % 2) + h
  auto sc = [&](const uint32_t (&d)[C::PLANES], int v) -> int {
    const int plane = FMT == 0 ? 0 : v / 2;
    const int byte = FMT == 0 ? 2 * v + h : 2 * (v % 2) + h;
    return (int)((d[plane] >> (8 * byte)) & 0xFFu);
  };

  // `mid(part, slots)` issues issue slot `part` of `slots` of the next step's
  // loads (part -1: all of them at once, as inactive waves do; part -2: its
  // grouped scale loads).
  // pin(): keeps a step's matrix instructions ahead of the barrier that
  // follows it where branches come next (the compiler would otherwise sink
  // them past it).
  auto pin = [&]() {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) asm volatile("" : "+a"(acc[i][j]));
  };
  // A wave whose rows of the tile all lie past its valid rows (a group's last,
  // partial tile; a masked slot's padding) only issues its share of the loads:
  // no fragment reads, no matrix instructions.  It meets every barrier and
  // runs the epilogue, whose stores then fall outside the tile's bounds.
  bool active = true;
  constexpr int kLoadRows = 4;
  constexpr bool kSch = EPI != kEpiDswigluQ;
  using Sc = Sched<FMT, GS, kSch>;
  // A tile's step 0 (kFirst) starts its accumulators from zero: its first
  // sub-step's matrix instructions take a zero accumulator operand, so the
  // accumulators are never cleared separately.  (A wave that skips its matrix
  // work keeps the previous tile's values; its stores are all out of bounds.)
  // `scl`: the step's scale words (row r of A at scl + r * RS, plane q at
  // + q * PS; B's rows from scl + BOFF).  `sync()`: the mid-step wait and
  // barrier of the MXFP8 schedule (every wave calls it once per step).
  auto step = [&](const uint8_t* cur, const uint8_t* scl, auto&& mid, auto&& sync, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    if (!active) {
      if constexpr (Sc::LATE) {     // the loads in slot order, so that the waits count alike
        mid(-2, 1);
#pragma unroll
        for (int s = 0; s < Sc::SYNC; ++s) mid(s, Sc::SLOTS);
        sync();
#pragma unroll
        for (int s = Sc::SYNC; s < Sc::SLOTS; ++s) mid(s, Sc::SLOTS);
      } else {
        mid(-1, 1);
      }
      return;
    }
    if constexpr (FMT == kNV) {
      // NVFP4: codes decode exactly to FP16 (E2M1 value x UE4M3 scale, at
      // most 6 significant bits, normal FP16 range) and multiply on the FP16
      // matrix cores, V_MFMA_F32_32X32X16_F16 (the BF16 rate).  A stage is 4 phases of 64 K; in phase q a
      // lane reads 16-byte chunk 2q + h of each fragment row (32 codes) and
      // scale dword q of the row (the 4 UE4M3 bytes of the phase's 16-groups;
      // this lane group's are bytes 2h and 2h + 1).  Sub-step u of the phase
      // multiplies codes 8u .. 8u + 7 of the lane's chunk (16-group 2h + u/2);
      // both operands use this same K order, so the products pair up.
      const uint8_t* la = cur + wm * WTM * SROW;
      const uint8_t* lb = cur + C::A_BYTES + wn * WTN * SROW;
      const uint8_t* lsa = scl + (wm * WTM + r32) * L::RS;
      const uint8_t* lsb = scl + L::BOFF + (wn * WTN + r32) * L::RS;
      uint4 ca[FI], cb[FJ], can[FI], cbn[FJ];
      uint32_t sa[FI], sb[FJ], san[FI], sbn[FJ];
      auto load_phase = [&](int q, uint4 (&xa)[FI], uint4 (&xb)[FJ], uint32_t (&ya)[FI], uint32_t (&yb)[FJ]) {
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          xa[i] = rd16(la, i, 2 * q);
          ya[i] = lds_read4(lsa + q * L::PS + 32 * i * L::RS);
        }
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          xb[j] = rd16(lb, j, 2 * q);
          yb[j] = lds_read4(lsb + q * L::PS + 32 * j * L::RS);
        }
      };
      auto word = [](const uint4& c, int u) -> uint32_t {
        return u == 0 ? c.x : (u == 1 ? c.y : (u == 2 ? c.z : c.w));
      };
      load_phase(0, ca, cb, sa, sb);
      mid(-2, 1);                     // the next step's scales, ahead of the matrix work
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q + 1 < 4) load_phase(q + 1, can, cbn, san, sbn);
        __builtin_amdgcn_sched_barrier(0);
        // this lane group's two UE4M3 scales per row (bit 7 ignored: unsigned)
        h2 fa[FI], fb[FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i)
          fa[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((sa[i] >> (16 * h)) & 0x7F7Fu, 1.0f, false);
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          fb[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((sb[j] >> (16 * h)) & 0x7F7Fu, 1.0f, false);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v8h da[FI], db[FJ];
#pragma unroll
          for (int i = 0; i < FI; ++i) da[i] = decode8(word(ca[i], u), fa[i][u >> 1]);
#pragma unroll
          for (int j = 0; j < FJ; ++j) db[j] = decode8(word(cb[j], u), fb[j][u >> 1]);
#pragma unroll
          for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  db[j], da[i], kFirst && q == 0 && u == 0 ? v16f{} : acc[i][j], 0, 0, 0);
              // the next step's loads: one slot after each MFMA of the first
              // sub-step (3 % faster than all at once ahead of it)
              if (q == 0 && u == 0) mid(i * FJ + j, FI * FJ);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (q + 1 < 4) {
#pragma unroll
          for (int i = 0; i < FI; ++i) {
            ca[i] = can[i];
            sa[i] = san[i];
          }
#pragma unroll
          for (int j = 0; j < FJ; ++j) {
            cb[j] = cbn[j];
            sb[j] = sbn[j];
          }
        }
      }
      return;
    }
    const uint8_t* la = cur + wm * WTM * SROW;
    const uint8_t* lb = cur + C::A_BYTES + wn * WTN * SROW;
    const uint8_t* lsa = scl + (wm * WTM + r32) * L::RS;
    const uint8_t* lsb = scl + L::BOFF + (wn * WTN + r32) * L::RS;
    if constexpr (Sc::LATE) {
      // MXFP8 with the load schedule above: groups (i, v) in i-major order.
      // The next group's A fragment is read during the current group; both
      // sub-steps' B fragments stay in registers (sub-step 1's are read
      // during group (0, 0)).
      Frag ga = rd(la, 0, 0);
      Frag gb[2][FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) gb[0][j] = rd(lb, j, 0);
      uint32_t gas[FI][C::PLANES], gbs[FJ][C::PLANES];
#pragma unroll
      for (int j = 0; j < FJ; ++j) gbs[j][0] = lds_read4(lsb + 32 * j * L::RS);
#pragma unroll
      for (int i = 0; i < FI; ++i) gas[i][0] = lds_read4(lsa + 32 * i * L::RS);
      mid(-2, 1);
#pragma unroll
      for (int i = 0; i < FI; ++i) {
#pragma unroll
        for (int v = 0; v < SUB; ++v) {
          if (8 * i + 4 * v == Sc::SYNC) sync();     // before row 1's A fragment is read
          Frag gan = ga;
          if (v == 0) gan = rd(la, i, 1);
          else if (i + 1 < FI) gan = rd(la, i + 1, 0);
          if (i == 0 && v == 0) {
#pragma unroll
            for (int j = 0; j < FJ; ++j) gb[1][j] = rd(lb, j, 1);
          }
          __builtin_amdgcn_sched_barrier(0);
          const v8i af = op(ga);
#pragma unroll
          for (int j = 0; j < FJ; ++j) {
            acc[i][j] = mfma32<FMT>(op(gb[v][j]), af, kFirst && v == 0 ? v16f{} : acc[i][j], sc(gbs[j], v),
                                    sc(gas[i], v));
            mid(8 * i + 4 * v + j, Sc::SLOTS);
          }
          __builtin_amdgcn_sched_barrier(0);
          ga = gan;
        }
      }
      return;
    }
    Frag fa = rd(la, 0, 0);
    Frag fb[FJ], fbn[FJ];
    fb[0] = rd(lb, 0, 0);
    uint32_t asc[FI][C::PLANES], bsc[FJ][C::PLANES];
#pragma unroll
    for (int q = 0; q < C::PLANES; ++q) {
#pragma unroll
      for (int j = 0; j < FJ; ++j) bsc[j][q] = lds_read4(lsb + q * L::PS + 32 * j * L::RS);
#pragma unroll
      for (int i = 0; i < FI; ++i) asc[i][q] = lds_read4(lsa + q * L::PS + 32 * i * L::RS);
    }
#pragma unroll
    for (int j = 1; j < FJ; ++j) fb[j] = rd(lb, j, 0);
    if constexpr (GS) mid(-2, 1);     // the next step's scales, ahead of the matrix work
#pragma unroll
    for (int v = 0; v < SUB; ++v) {
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        Frag fan = fa;
        if (i + 1 < FI) fan = rd(la, i + 1, v);
        else if (v + 1 < SUB) fan = rd(la, 0, v + 1);
        if (v + 1 < SUB && i < FJ) fbn[i] = rd(lb, i, v + 1);
        __builtin_amdgcn_sched_barrier(0);
        const v8i af = op(fa);
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          acc[i][j] = mfma32<FMT>(op(fb[j]), af, kFirst && v == 0 ? v16f{} : acc[i][j], sc(bsc[j], v),
                                  sc(asc[i], v));
          // the next step's loads ride between the MFMAs of the first kLoadRows
          // rows, one issue slot after each (measured: 3 % faster than issuing
          // them all ahead of one row; the wave that stalls on a full address
          // queue then stalls with a matrix instruction in flight)
          if (4 * v + i < kLoadRows) mid((4 * v + i) * FJ + j, kLoadRows * FJ);
        }
        __builtin_amdgcn_sched_barrier(0);
        fa = fan;
      }
      if (v + 1 < SUB) {
#pragma unroll
        for (int j = 0; j < FJ; ++j) fb[j] = fbn[j];
      }
    }
  };

  Tile tl = make_tile<FMT>(p, tt, total_gm, n_heavy, NT, mt_per, nk, t, kunit, TCOLS, sk_first.a, sk_first.b);
  int st = 0;                                   // stage of the current step
  // first tile: steps 0 and 1 in flight, wait for step 0
  const uint32_t smem_lds = ufirst(lds_addr(smem));      // LDS byte address of stage 0
  issue<FMT, GS, PAIRED, kSch, NTB>(tl, lo, 0, smem_lds, smem_lds, w);
  issue<FMT, GS, PAIRED, kSch, NTB>(tl, lo, 1, smem_lds + L::STAGE, smem_lds, w);
  wait_vm<L::OPS1>();
  bar();
  // the scale words of step k of tile `tl` in stage `stage`
  auto scl = [&](const Tile& tt_, int k, int stage) -> const uint8_t* {
    if constexpr (GS)
      return smem + 2 * L::STAGE + ((tt_.sg + k / L::SPG) & 1) * L::SBUF + (k % L::SPG) * C::PLANES * 4;
    else
      return smem + stage * L::STAGE + C::A_BYTES + C::B_BYTES;
  };

  // cleared once, so that a wave without matrix work in its first tile
  // stores defined values (out of bounds, dropped)
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Stream-K pieces (kEpiStream).  Every piece stores its accumulators as an
  // FP32 partial tile -- 16-byte chunks in lane order, chunk q of thread x at
  // (q * THREADS + x) * 16 -- in a slot of this workgroup: a piece that ends
  // its tile (the owner, always a workgroup's last piece) in slot `slot` of
  // the second half of the partial area, which only this workgroup reads
  // back (after its tile loop, sk_reduce); any other piece in slot `slot` of
  // the first half, whose flag it then raises for the tile's owner.  Those
  // partials and the flags take agent-scope (sc1) accesses, which bypass the
  // non-coherent caches between the XCDs, and a flag is raised only after
  // the workgroup's partial stores have completed (vmcnt 0 in every wave,
  // then the barrier).  A flag holds the call's tag in its low word and the
  // tag's complement in its high word, so that left-over workspace contents
  // are not taken for it.
  typedef uint32_t sk_v4u __attribute__((ext_vector_type(4)));
  constexpr int kSc0 = 1, kSc1 = 16;                // cache policies: L1 bypass, agent scope
  constexpr uint32_t kSkSlot = (uint32_t)BM * BN * 4;
  auto sk_flag = [&]() { return ((uint64_t)(~p.sk_tag) << 32) | p.sk_tag; };
  auto sk_handoff = [&](const Tile& pc) -> bool {
    if constexpr (SKM) {
      static_assert(FI * FJ * 4 * C::THREADS * 16 == BM * BN * 4, "a partial slot holds one tile");
      const bool owner = pc.sk1 == upt;
      float* base = p.partial + ((owner ? (int64_t)stride : 0) + slot) * (int64_t)(BM * BN);
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)kSkSlot, 0x00020000);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t off = (uint32_t)((((i * FJ + j) * 4 + b) * C::THREADS + tid) * 16);
            const sk_v4u o = sk_v4u{__float_as_uint(acc[i][j][4 * b]), __float_as_uint(acc[i][j][4 * b + 1]),
                                    __float_as_uint(acc[i][j][4 * b + 2]), __float_as_uint(acc[i][j][4 * b + 3])};
            if (owner) __builtin_amdgcn_raw_buffer_store_b128(o, prs, (int)off, 0, 0);
            else __builtin_amdgcn_raw_buffer_store_b128(o, prs, (int)off, 0, kSc1);
          }
      if (!owner) {
        wait_vm<0>();
        bar();
        if (tid == 0) __hip_atomic_store(p.sk_flags + slot, sk_flag(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return true;
    }
    return false;
  };
  // The owner's reduction, after its tile loop (a workgroup ends at most one
  // tile: its run is shorter than a tile): waits for the flags of the
  // workgroups of its group that ran the tile's earlier units, if any (lower
  // indices: those waits end; a wait that still outlasts kSkSpin polls gives
  // up and sets the timeout word, so that a fault elsewhere leaves a wrong
  // tile, not a hung GPU), adds their partials in K order and then its own,
  // applies bias / alpha, rounds once and stores 4 columns per chunk; then
  // clears the flags.
  auto sk_reduce = [&]() {
    if constexpr (SKM) {
      const SkRun rn = sk_run();
      const Piece pc = piece(rn.u1 > rn.u0 && (rn.u1 - 1) / upt > rn.u0 / upt ? 1 : 0);
      if (pc.t >= total || pc.b != upt) return;
      const Tile tt_ = make_tile<FMT>(p, tt, total_gm, n_heavy, NT, mt_per, nk, pc.t, kunit, TCOLS, pc.a, pc.b);
      // the slot of the group's workgroup that holds the tile's first unit
      const int64_t ut = rn.u0 - pc.a - rn.g0;
      const int c_first = rn.base + (int)(((ut + 1) * per_xcd + rn.gu - 1) / rn.gu) - 1;
      wait_vm<0>();                                      // this workgroup's own partial
      if (tid == 0) {
        for (int c = c_first; c < slot; ++c) {
          int n = 0;
          while (__hip_atomic_load(p.sk_flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != sk_flag()) {
            if (++n >= kSkSpin) {
              __hip_atomic_store(p.sk_flags + kSkMaxGrid, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
      }
      bar();
      asm volatile("" ::: "memory");                     // the partial loads stay behind the wait
      const __amdgpu_buffer_rsrc_t own = __builtin_amdgcn_make_buffer_rsrc(
          p.partial + ((int64_t)stride + slot) * (int64_t)(BM * BN), (short)0, (int)kSkSlot, 0x00020000);
      const uint8_t* obase = uniform_ptr(reinterpret_cast<const uint8_t*>(p.out + tt_.row0 * p.n));
      const uint32_t obytes = ufirst((uint32_t)((tt_.row_end - tt_.row0) * p.n * 2));
      const __amdgpu_buffer_rsrc_t orsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(obase), (short)0, (int)obytes, 0x00020000);
      const uint16_t* bias = p.bias ? p.bias + (int64_t)tt_.g * p.n : nullptr;
      const float alpha = FMT == kNV ? p.alpha[tt_.g] : 1.0f;
      const bool f16o = p.out_f16 != 0;
      constexpr int kQ = FI * FJ * 4, kBatch = 8;
      for (int q0 = 0; q0 < kQ; q0 += kBatch) {
        float f[kBatch][4];
#pragma unroll
        for (int e = 0; e < kBatch; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) f[e][r] = 0.f;
        for (int c = c_first; c < slot; ++c) {
          const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
              p.partial + (int64_t)c * (BM * BN), (short)0, (int)kSkSlot, 0x00020000);
          sk_v4u v[kBatch];
#pragma unroll
          for (int e = 0; e < kBatch; ++e)
            v[e] = __builtin_bit_cast(sk_v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                                  prs, (int)(((q0 + e) * C::THREADS + tid) * 16), 0, kSc1));
#pragma unroll
          for (int e = 0; e < kBatch; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) f[e][r] += __uint_as_float(v[e][r]);
        }
        sk_v4u w[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e)
          w[e] = __builtin_bit_cast(sk_v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                                own, (int)(((q0 + e) * C::THREADS + tid) * 16), 0, kSc0));
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
          // chunk q = (i FJ + j) 4 + b: fragment (i, j), columns 8 b + 4 h .. + 3
          const int q = q0 + e, i = q / (FJ * 4), j = (q / 4) % FJ, b = q % 4;
          const int64_t mr = wm * WTM + i * 32 + r32;
          const int64_t n = tt_.n0 + wn * WTN + j * 32 + 8 * b + 4 * h;
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = f[e][r] + __uint_as_float(w[e][r]);
          if (bias != nullptr && n < p.n) {
            const uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
            x[0] += bf16_lo(bb.x);
            x[1] += bf16_hi(bb.x);
            x[2] += bf16_lo(bb.y);
            x[3] += bf16_hi(bb.y);
          }
          if (FMT == kNV)
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] *= alpha;
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          const v2u o = f16o ? v2u{pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3])}
                             : v2u{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          const uint32_t off = n < p.n ? (uint32_t)((mr * p.n + n) * 2) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b64(o, orsrc, (int)off, 0, 0);
        }
      }
      if (tid == 0)
        for (int c = c_first; c < slot; ++c)
          __hip_atomic_store(p.sk_flags + c, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  bool prior_stores = false;
  while (true) {
    active = wm * WTM < tl.row_end - tl.row0;

    // Steps 0 .. nk-2.  Step 1's loads were issued with step 0's, before the
    // previous tile's stores; step k >= 1 issues step k + 1 into the stage
    // step k - 1 used.
    // step 0: step 1's loads were issued with step 0's, before the previous
    // tile's stores, which stay in flight
    step(smem + st * L::STAGE, scl(tl, 0, st), [](int, int) {}, []() {}, std::true_type{});
    pin();
    __builtin_amdgcn_sched_barrier(0);
    if (prior_stores) wait_vm<kStores>();
    else wait_vm<0>();
    bar();
    st ^= 1;
    for (int k = 1; k + 1 < tl.nk; ++k) {
      const uint32_t nxt = smem_lds + (st ^ 1) * L::STAGE;
      step(smem + st * L::STAGE, scl(tl, k, st),
           [&](int part, int slots) { issue<FMT, GS, PAIRED, kSch, NTB>(tl, lo, k + 1, nxt, smem_lds, w, part, slots); },
           [&]() {
             // this step's late loads, issued in step k - 1 (step 1's loads
             // were issued whole ahead of the tile and have landed): since
             // then this step issued its scale loads, if any, and the
             // EARLY_BEFORE_SYNC loads of the slots before SYNC
             if (k >= 2) {
               wait_vm<Sc::EARLY_BEFORE_SYNC>();
               bar();
             }
           },
           std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<Sc::LATE ? Sc::N_LATE : 0>();     // all but the late loads of step k + 1
      bar();
      st ^= 1;
    }
    // last step: the next tile's step 0 goes into the other stage
    // (stream-K: the second piece after the first, read from LDS, whose
    // store the first piece's barriers have long ordered)
    const Piece pn = !SKM ? Piece{tile_of(round + 1), 0, 0}
                          : (round == 0 ? Piece{__builtin_amdgcn_readfirstlane(sk_second[0]),
                                                __builtin_amdgcn_readfirstlane(sk_second[1]),
                                                __builtin_amdgcn_readfirstlane(sk_second[2])}
                                        : Piece{total, 0, 0});
    const int t_next = pn.t;
    const bool has_next = t_next < tile_end;
    Tile tn = tl;
    if (has_next) {
      tn = make_tile<FMT>(p, tt, total_gm, n_heavy, NT, mt_per, nk, t_next, kunit, TCOLS, pn.a, pn.b);
      // the scale buffer after this tile's last scale group
      tn.sg = (tl.sg + tl.nk / L::SPG) & 1;
      issue<FMT, GS, PAIRED, kSch, NTB>(tn, lo, 0, smem_lds + (st ^ 1) * L::STAGE, smem_lds, w);
    }
    step(smem + st * L::STAGE, scl(tl, tl.nk - 1, st), [](int, int) {},
         [&]() {
           // the late loads of this step (issued in step nk - 2 >= 1) are
           // followed only by the next tile's step-0 loads
           if (tl.nk >= 3) {
             if (has_next) wait_vm<2 * C::LOADS + L::SCALE_OPS>();
             else wait_vm<0>();
             bar();
           }
         },
         std::false_type{});
    pin();
    bar();                            // stage `st` is free
    if (has_next) issue<FMT, GS, PAIRED, kSch, NTB>(tn, lo, 1, smem_lds + st * L::STAGE, smem_lds, w);

    if constexpr (EPI == kEpiSplit) {
      // ---- K-split epilogue: this slice's FP32 partial tile to
      // partial[slice][row][col], 16-byte buffer stores of 4 consecutive
      // columns (lane l, register 4b + r holds fragment row l % 32, column
      // 8b + 4(l/32) + r); rows past the tile end fall outside the
      // descriptor, columns past n take the drop marker.
      const uint8_t* pb = uniform_ptr(reinterpret_cast<const uint8_t*>(
          p.partial + ((int64_t)tl.slice * p.m_rows + tl.row0) * p.n));
      const uint32_t pbytes = ufirst((uint32_t)((tl.row_end - tl.row0) * p.n * 4));
      const __amdgpu_buffer_rsrc_t prsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pb), (short)0, (int)pbytes, 0x00020000);
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          const int64_t mr = wm * WTM + i * 32 + r32;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int64_t n = tl.n0 + wn * WTN + j * 32 + 8 * b + 4 * h;
            const uint32_t off = n < p.n ? (uint32_t)((mr * p.n + n) * 4) : 0x80000000u;
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u o = v4u{__float_as_uint(acc[i][j][4 * b]), __float_as_uint(acc[i][j][4 * b + 1]),
                              __float_as_uint(acc[i][j][4 * b + 2]), __float_as_uint(acc[i][j][4 * b + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(o, prsrc, (int)off, 0, 0);
          }
        }
    } else if constexpr (DSW) {
      // ---- dSwiGLU epilogue (cuDNN FE "Grouped GEMM + dGLU (SM100)", Step 2,
      // dSwiGLU).  Fragment (i, j) of this wave holds R columns
      // nb = n0 + wn WTN + 32 j + [0, 32) -- one 32-column block pair of C and D,
      // columns 2 nb (input) and 2 nb + 32 (gate) -- for rows 32 i + [0, 32):
      // lane l, register 4b + r is row l % 32, column 8b + 4(l/32) + r; lanes
      // l and l ^ 32 swap quads so that each lane owns two runs of 8
      // consecutive columns, 16e + 8(l/32) .. + 7.  With X = beta C (the
      // group's beta) and R times the group's alpha^2:
      //   s = sigmoid(gate), swish = gate s,
      //   D[input] = R prob swish,  D[gate] = R prob input s (1 + gate (1 - s)),
      //   dprob[row] += sum of swish input R over the row's columns
      // in FP32, D rounded once to BF16.  The row sums of a wave's columns are
      // added to dprob with one atomic per row and wave.  Rows past the tile's
      // rows and columns past n fall outside the buffer bounds (loads read 0,
      // stores are dropped) and add nothing to dprob.
      const int64_t C2 = 2 * p.n;
      const int64_t trows = tl.row_end - tl.row0;
      const uint32_t cbytes = ufirst((uint32_t)(trows * C2 * 2));
      const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(uniform_ptr(reinterpret_cast<const uint8_t*>(p.c_in + tl.row0 * C2))), (short)0,
          (int)cbytes, 0x00020000);
      // BF16 D, or (kEpiDswigluQ) its MXFP8 codes [rows, 2n] and UE8M0
      // scales [rows, 2n / 32]: per row, each 32-column block of D (one input
      // or gate block) is one scale group, quantised from the BF16 values
      // with the rule of hq_group_wise_quant
      const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(uniform_ptr(EPI == kEpiDswigluQ
                                               ? p.q_out + tl.row0 * C2
                                               : reinterpret_cast<const uint8_t*>(p.d_out + tl.row0 * C2))),
          (short)0, (int)(EPI == kEpiDswigluQ ? cbytes / 2 : cbytes), 0x00020000);
      const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(uniform_ptr(EPI == kEpiDswigluQ ? p.sf_out + tl.row0 * (C2 / 32) : p.sf_out)),
          (short)0, (int)(EPI == kEpiDswigluQ ? cbytes / 64 : 0), 0x00020000);
      const float al = p.alpha != nullptr ? p.alpha[tl.g] : 1.0f;
      const float a2 = al * al;
      const float be = p.beta != nullptr ? p.beta[tl.g] : 1.0f;
      // lane-derived offsets from an opaque copy of the lane id (computed
      // here, not kept live through the K loop)
      int le;
      asm volatile("v_mov_b32 %0, %1" : "=v"(le) : "v"(lane));
      const int he = le >> 5, re = le & 31;
      typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int64_t mr = wm * WTM + i * 32 + re;             // row within the tile
        const bool row_ok = mr < trows;
        const float pr = row_ok ? p.prob[tl.row0 + mr] : 0.0f;
        // the C runs of every fragment of the row: input and gate, 16 bytes
        // each (the quantising epilogue loads them fragment by fragment: its
        // codes and scales need more registers)
        v4u cin[FJ][2], cgt[FJ][2];
        uint32_t coff[FJ][2];
        auto load_c = [&](int j) {
          const int64_t nb = tl.n0 + wn * WTN + j * 32;        // first R column of the pair
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int64_t col = 2 * nb + 16 * e + 8 * he;       // C / D column of the input run
            coff[j][e] = nb < p.n ? (uint32_t)((mr * C2 + col) * 2) : 0x80000000u;
            cin[j][e] = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)coff[j][e], 0, 0);
            cgt[j][e] = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)(coff[j][e] + 64u), 0, 0);
          }
        };
        if constexpr (EPI == kEpiDswiglu) {
#pragma unroll
          for (int j = 0; j < FJ; ++j) load_c(j);
        }
        float dsum = 0.0f;
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          if constexpr (EPI == kEpiDswigluQ) load_c(j);
          uint32_t din[2][4], dgt[2][4];       // BF16 pairs of the lane's two runs
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float run[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][8 * e + r]),
                                                               __float_as_uint(acc[i][j][8 * e + 4 + r]), false, false);
              run[r] = __uint_as_float(sw[0]);
              run[4 + r] = __uint_as_float(sw[1]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float dv[2], gv[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int t = 2 * q + u;
                const uint32_t wi = cin[j][e][q], wg = cgt[j][e][q];
                const float xi = be * (u == 0 ? bf16_lo(wi) : bf16_hi(wi));
                const float xg = be * (u == 0 ? bf16_lo(wg) : bf16_hi(wg));
                const float r = run[t] * a2;
                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-xg * 1.4426950408889634f));
                const float swish = xg * sg;
                const float rp = r * pr;
                dv[u] = rp * swish;
                gv[u] = rp * xi * sg * (1.0f + xg * (1.0f - sg));
                dsum += coff[j][e] != 0x80000000u ? swish * xi * r : 0.0f;
              }
              din[e][q] = pack_bf16x2(dv[0], dv[1]);
              dgt[e][q] = pack_bf16x2(gv[0], gv[1]);
            }
            if constexpr (EPI == kEpiDswiglu) {
              __builtin_amdgcn_raw_buffer_store_b128(v4u{din[e][0], din[e][1], din[e][2], din[e][3]}, drs,
                                                     (int)coff[j][e], 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(v4u{dgt[e][0], dgt[e][1], dgt[e][2], dgt[e][3]}, drs,
                                                     (int)(coff[j][e] + 64u), 0, 0);
            }
          }
          if constexpr (EPI == kEpiDswigluQ) {
            // the block's amax over this lane's two runs and lane l ^ 32's,
            // on the BF16 bit patterns (|x| of the upper half is bits & 0x7fff0000)
            uint32_t ai = 0, ag = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t i0 = (din[e][q] << 16) & 0x7fffffffu, i1 = din[e][q] & 0x7fff0000u;
                const uint32_t g0 = (dgt[e][q] << 16) & 0x7fffffffu, g1 = dgt[e][q] & 0x7fff0000u;
                ai = i0 > ai ? i0 : ai;
                ai = i1 > ai ? i1 : ai;
                ag = g0 > ag ? g0 : ag;
                ag = g1 > ag ? g1 : ag;
              }
            const uint32_t oi = (uint32_t)__shfl_xor((int)ai, 32, 64);
            const uint32_t og = (uint32_t)__shfl_xor((int)ag, 32, 64);
            ai = oi > ai ? oi : ai;
            ag = og > ag ? og : ag;
            const uint32_t sbi = mx_scale_byte<8>(ai), sbg = mx_scale_byte<8>(ag);
            typedef uint32_t v2u __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              float vi[8], vg[8];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                vi[2 * q] = bf16_lo(din[e][q]);
                vi[2 * q + 1] = bf16_hi(din[e][q]);
                vg[2 * q] = bf16_lo(dgt[e][q]);
                vg[2 * q + 1] = bf16_hi(dgt[e][q]);
              }
              // code bytes sit at half the BF16 byte offset (drop marker kept)
              const uint32_t qo = coff[j][e] == 0x80000000u ? 0x80000000u : coff[j][e] / 2;
              const uint2 ci = mx_fp8x8(vi, sbi), cg = mx_fp8x8(vg, sbg);
              __builtin_amdgcn_raw_buffer_store_b64(v2u{ci.x, ci.y}, drs, (int)qo, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b64(v2u{cg.x, cg.y}, drs, (int)(qo + 32u), 0, 0);
            }
            // scale bytes of the input and gate blocks from lane group 0 (the
            // other group's stores take the drop marker)
            const int64_t nb = tl.n0 + wn * WTN + j * 32;
            const uint32_t so = he == 0 && nb < p.n ? (uint32_t)(mr * (C2 / 32) + nb / 16) : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbi, srs, (int)so, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbg, srs, (int)(so == 0x80000000u ? so : so + 1u), 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the row's other 16 columns of every fragment are in lane l ^ 32
        dsum += __shfl_xor(dsum, 32, 64);
        if (row_ok && he == 0) unsafeAtomicAdd(p.dprob + tl.row0 + mr, dsum);
        // one fragment row at a time (all rows' loads at once run out of registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (EPI == kEpiSwiglu) {
      // ---- SwiGLU + MXFP8 re-quant epilogue.  Fragment j < 2 of this wave
      // holds gate and fragment j + 2 up of the same 32 y columns
      // (ycol .. ycol + 31, one 32-group), in the same lanes and registers:
      // lane l, register 4b + r is row l % 32, column 8b + 4(l/32) + r.  Each
      // value gets the bias and the BF16 rounding of the gate|up output, then
      // y = up * silu(gate) and the quantiser of hq_group_wise_quant -- the
      // same instructions as the separate GEMM and SwiGLU kernels, so the
      // codes are the same.  Rows at or past the group's valid rows fall
      // outside the store descriptors.
      const int64_t H = p.h;
      const int64_t vrows = tl.vend > tl.row0 ? tl.vend - tl.row0 : 0;
      const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(uniform_ptr(p.q_out + tl.row0 * H)), (short)0,
          (int)ufirst((uint32_t)(vrows * H)), 0x00020000);
      const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(uniform_ptr(p.sf_out + tl.row0 * (H / 32))), (short)0,
          (int)ufirst((uint32_t)(vrows * (H / 32))), 0x00020000);
      const uint16_t* bias = !NOBIAS && p.bias ? p.bias + (int64_t)tl.g * p.n : nullptr;
      // lane-derived offsets from an opaque copy of the lane id, so that the
      // compiler computes them here instead of keeping them live through the
      // K loop (which runs out of registers)
      int le;
      asm volatile("v_mov_b32 %0, %1" : "=v"(le) : "v"(lane));
      const int he = le >> 5, re = le & 31;
      const uint32_t H32 = (uint32_t)H;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t ycol = tl.n0 + wn * 64 + 32 * j;          // the 32-group's first column
        // this lane's gate and up bias of the fragment pair's columns
        float gb[4][4], ub[4][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t col = ycol + 8 * b + 4 * he;
          uint2 bg = make_uint2(0u, 0u), bu = make_uint2(0u, 0u);
          if (bias != nullptr) {
            bg = *reinterpret_cast<const uint2*>(bias + col);
            bu = *reinterpret_cast<const uint2*>(bias + H + col);
          }
          gb[b][0] = bf16_lo(bg.x); gb[b][1] = bf16_hi(bg.x); gb[b][2] = bf16_lo(bg.y); gb[b][3] = bf16_hi(bg.y);
          ub[b][0] = bf16_lo(bu.x); ub[b][1] = bf16_hi(bu.x); ub[b][2] = bf16_lo(bu.y); ub[b][3] = bf16_hi(bu.y);
        }
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          const uint32_t mr = (uint32_t)(wm * WTM + i * 32 + re);   // row within the tile
          float y[4][4];
          uint32_t amax = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              uint32_t g2, u2;
              if constexpr (NOBIAS) {
                g2 = pack_bf16x2(acc[i][j][4 * b + r], acc[i][j][4 * b + r + 1]);
                u2 = pack_bf16x2(acc[i][j + 2][4 * b + r], acc[i][j + 2][4 * b + r + 1]);
              } else {
                g2 = pack_bf16x2(acc[i][j][4 * b + r] + gb[b][r], acc[i][j][4 * b + r + 1] + gb[b][r + 1]);
                u2 = pack_bf16x2(acc[i][j + 2][4 * b + r] + ub[b][r], acc[i][j + 2][4 * b + r + 1] + ub[b][r + 1]);
              }
              y[b][r] = silu_mul(bf16_lo(g2), bf16_lo(u2));
              y[b][r + 1] = silu_mul(bf16_hi(g2), bf16_hi(u2));
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t a = __float_as_uint(y[b][r]) & 0x7fffffffu;
              amax = a > amax ? a : amax;
            }
          }
          // the other 16 columns of the group are in lane l ^ 32
          const uint32_t other = (uint32_t)__shfl_xor((int)amax, 32, 64);
          amax = other > amax ? other : amax;
          const uint32_t sb = mx_scale_byte<8>(amax);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            // lanes l and l ^ 32 swap a quad: this lane's 8-column run
            // ycol + 16e + 8(l/32) .. + 7
            float run[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[2 * e][r]),
                                                               __float_as_uint(y[2 * e + 1][r]), false, false);
              run[r] = __uint_as_float(sw[0]);
              run[4 + r] = __uint_as_float(sw[1]);
            }
            const uint2 codes = mx_fp8x8(run, sb);
            const uint32_t c0 = (uint32_t)ycol + 16 * e + 8 * he;
            typedef uint32_t v2u __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(v2u{codes.x, codes.y}, qrs, (int)(mr * H32 + c0), 0, 0);
            if (p.y_debug != nullptr) {
              const uint8_t* ybase = uniform_ptr(reinterpret_cast<const uint8_t*>(p.y_debug + tl.row0 * H));
              const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
                  const_cast<uint8_t*>(ybase), (short)0, (int)ufirst((uint32_t)(vrows * H * 4)), 0x00020000);
              typedef uint32_t v4u __attribute__((ext_vector_type(4)));
              const uint32_t yo = (mr * H32 + c0) * 4;
              __builtin_amdgcn_raw_buffer_store_b128(
                  v4u{__float_as_uint(run[0]), __float_as_uint(run[1]), __float_as_uint(run[2]), __float_as_uint(run[3])},
                  yrs, (int)yo, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(
                  v4u{__float_as_uint(run[4]), __float_as_uint(run[5]), __float_as_uint(run[6]), __float_as_uint(run[7])},
                  yrs, (int)(yo + 16), 0, 0);
            }
          }
          // the scale byte from lane group 0 (lane group 1's store takes the
          // drop marker: one store instruction for the wave either way)
          const uint32_t so = he == 0 ? mr * (H32 / 32) + (uint32_t)ycol / 32 : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, srs, (int)so, 0, 0);
          // one 32-group at a time (interleaving the groups runs out of registers)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else if (sk_handoff(tl)) {
      // a stream-K piece that does not end its tile: its partial is handed off
    } else {
      // ---- epilogue: BF16 (+bias), 16-byte buffer stores relative to the
      // tile's first row.  32x32 result: lane l holds D[8b + 4(l/32) + r][l%32]
      // in register 4b + r, i.e. out[m = l%32][n = 8b + 4(l/32) + r].  Lanes l
      // and l^32 swap one 4-column quad so each lane owns 8 consecutive
      // columns: lane group 0 stores columns 8b..8b+7 for b = 0, 2 and lane
      // group 1 for b = 1, 3.
      const uint8_t* obase = uniform_ptr(reinterpret_cast<const uint8_t*>(p.out + tl.row0 * p.n));
      const uint32_t obytes = ufirst((uint32_t)((tl.row_end - tl.row0) * p.n * 2));
      const __amdgpu_buffer_rsrc_t orsrc =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(obase), (short)0, (int)obytes, 0x00020000);
      const uint16_t* bias = p.bias ? p.bias + (int64_t)tl.g * p.n : nullptr;
      const float alpha = FMT == kNV ? p.alpha[tl.g] : 1.0f;   // NVFP4: g_A * g_B per group
      constexpr bool F16O = EPI == kEpiF16;                    // binary16 instead of BF16
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        v4f bq[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t n = tl.n0 + wn * WTN + j * 32 + 8 * b + 4 * h;
          bq[b] = v4f{0.f, 0.f, 0.f, 0.f};
          if (bias != nullptr && n < p.n) {
            uint2 bb = *reinterpret_cast<const uint2*>(bias + n);
            bq[b] = v4f{bf16_lo(bb.x), bf16_hi(bb.x), bf16_lo(bb.y), bf16_hi(bb.y)};
          }
        }
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          const int64_t mr = wm * WTM + i * 32 + r32;            // row within the tile
          uint32_t pk[4][2];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              f[r] = FMT == kNV ? acc[i][j][4 * b + r] * alpha : acc[i][j][4 * b + r] + bq[b][r];
            pk[b][0] = F16O ? pack_f16x2(f[0], f[1]) : pack_bf16x2(f[0], f[1]);
            pk[b][1] = F16O ? pack_f16x2(f[2], f[3]) : pack_bf16x2(f[2], f[3]);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {            // e = 0: quads b = 0/1, e = 1: b = 2/3
            const int bl = 2 * e, bh = 2 * e + 1;
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            v4u o;
            if constexpr (FMT != kNV) {
              // V_PERMLANE32_SWAP(x = quad 2e, y = quad 2e+1) leaves
              // x = {x[0..31], y[0..31]} and y = {x[32..63], y[32..63]}: in
              // either lane group (x, y) are then the first and second four
              // columns of the lane's 8-column run
              const auto sw0 = __builtin_amdgcn_permlane32_swap(pk[bl][0], pk[bh][0], false, false);
              const auto sw1 = __builtin_amdgcn_permlane32_swap(pk[bl][1], pk[bh][1], false, false);
              o = v4u{sw0[0], sw1[0], sw0[1], sw1[1]};
            } else {
              // (NVFP4 keeps the LDS-routed exchange: with the swap its kernel
              // runs out of registers)  group 0 receives the partner's b = 2e
              // quad, group 1 the partner's b = 2e+1 quad
              const uint32_t r0 = (uint32_t)__shfl_xor((int)(h == 0 ? pk[bh][0] : pk[bl][0]), 32, 64);
              const uint32_t r1 = (uint32_t)__shfl_xor((int)(h == 0 ? pk[bh][1] : pk[bl][1]), 32, 64);
              o = h == 0 ? v4u{pk[bl][0], pk[bl][1], r0, r1} : v4u{r0, r1, pk[bh][0], pk[bh][1]};
            }
            const int64_t n = tl.n0 + wn * WTN + j * 32 + 8 * (h == 0 ? bl : bh);
            const uint32_t off = n < p.n ? (uint32_t)((mr * p.n + n) * 2) : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b128(o, orsrc, (int)off, 0, 0);
          }
        }
      }
    }
    if (!has_next) break;
    // the next tile's step 0 was issued before its step 1 (nk > 1) and these
    // kStores stores
    wait_vm<L::OPS1 + kStores>();
    bar();
    t = t_next;
    ++round;
    tl = tn;
    st ^= 1;
    prior_stores = true;
  }
  sk_reduce();
}

// Sums the K-split partial tiles slice by slice, in slice order, and writes
// the BF16 output with the bias (MX) or alpha (NVFP4) of the row's group:
// the same arithmetic as the single-pass epilogue on the summed tile.  Block
// b takes rows b, b + grid, ...; its threads walk the row's 4-column chunks
// (n % 8 == 0).
__global__ __launch_bounds__(256) void splitk_reduce(GemmArgs p) {
  const int64_t plane = p.m_rows * p.n;          // floats per slice
  const int64_t chunks = p.n / 4;
  const int64_t ldo = p.ldo > 0 ? p.ldo : p.n;
  for (int64_t row = blockIdx.x; row < p.m_rows; row += gridDim.x) {
    const int64_t g = row / p.slot_rows;
    const float alpha = p.mode == kNVFP4 ? p.alpha[g] : 1.0f;
    const uint16_t* bias = p.bias ? p.bias + g * p.n : nullptr;
    for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
      const int64_t e = row * p.n + 4 * c;
      v4f v = *reinterpret_cast<const v4f*>(p.partial + e);
      for (int sl = 1; sl < p.ksplit; ++sl) v += *reinterpret_cast<const v4f*>(p.partial + sl * plane + e);
      float f[4];
      if (p.mode == kNVFP4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = v[r] * alpha;
      } else if (bias != nullptr) {
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + 4 * c);
        f[0] = v[0] + bf16_lo(bb.x);
        f[1] = v[1] + bf16_hi(bb.x);
        f[2] = v[2] + bf16_lo(bb.y);
        f[3] = v[3] + bf16_hi(bb.y);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) f[r] = v[r];
      }
      *reinterpret_cast<uint2*>(p.out + row * ldo + 4 * c) =
          p.out_f16 ? make_uint2(pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]))
                    : make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
    }
  }
}

// Compute units a launch may use (cu_limit caps them).
int plan_cus(const GemmArgs& p, const DeviceInfo& dev) {
  int cus = dev.num_cus;
  if (p.cu_limit > 0 && p.cu_limit < cus) cus = p.cu_limit;
  return cus;
}

}  // namespace

// The split plan of a dense or batch call (uniform form) on the tiled kernel;
// the launcher follows it when the caller's workspace holds sp.bytes.
//  * Tail split (dense form): when the tiles fill some rounds of the grid and
//    leave a last round at most half full, that round's tiles -- the last ones
//    in the tile order, a rectangle of whole n-tile columns of the last block
//    of 4 m-tiles -- run as a second, K-split launch on the rectangle, so they
//    occupy the CUs with S times smaller units.  It pays only when a tile is
//    long next to writing and summing its S partial planes: at least about
//    110 us of matrix work per tail tile on a loaded chip, i.e. 40 FP4 steps,
//    48 FP8 steps or 12 NVFP4 steps (whose FP16 products are slower).
//  * Stream-K (dense form) where the tiles make one round of more than a
//    third of the grid: the K units (of at least two steps, on scale-group
//    boundaries) of all tiles are dealt out in equal runs, one per
//    workgroup, when the longest run is at most 0.7 of a tile's units and
//    saves enough matrix time to pay for the FP32 hand-off (below).
//  * K split (dense and batch forms) where the tiles cannot fill half of the
//    CUs: S slices of at least 4 K steps each, S * tiles <= CUs, at most 8,
//    when the steps saved pay for the partial planes (below).
// Every plan's FP32 partials follow the kWsHeader bytes of stream-K flags.
SplitPlan plan_split(const GemmArgs& p, const DeviceInfo& dev) {
  SplitPlan sp{};
  sp.kind = kSplitNone;
  if (p.form != kUniform || p.n * 1024 >= ((int64_t)1 << 31)) return sp;
  const int64_t NT = (p.n + BN - 1) / BN;
  const int64_t total_gm = (int64_t)p.num_groups * ((p.slot_rows + BM - 1) / BM);
  const int64_t tiles = total_gm * NT;
  const int cus = plan_cus(p, dev);
  const int64_t grid_full = cus >= 8 ? cus - cus % 8 : cus;
  const int64_t nk = p.lda / SROW;
  const int64_t kTailMinSteps = p.mode == kNVFP4 ? 12 : (p.mode == kMXFP8 ? 48 : 40);
  if (p.num_groups == 1 && tiles > grid_full && nk >= kTailMinSteps) {
    const int64_t tail = tiles % grid_full;
    const int64_t last_blk = (total_gm - 1) / kMB;
    const int64_t mb = total_gm - last_blk * kMB;         // m-tiles of the last block
    const int64_t cols = (tail + mb - 1) / mb;            // n-tile columns of the rectangle
    int64_t S = cols * mb > 0 ? grid_full / (cols * mb) : 0;
    if (S > nk / 4) S = nk / 4;
    if (S > 8) S = 8;
    if (tail > 0 && tail * 2 <= grid_full && cols < NT && S >= 2) {
      sp.kind = kSplitTail;
      sp.S = S;
      sp.r0 = last_blk * kMB * BM;
      sp.c0 = (NT - cols) * BN;
      sp.rect_tiles = cols * mb;
      sp.bytes = kWsHeader + (uint64_t)(S * (p.m_rows - sp.r0) * (p.n - sp.c0) * 4);
    }
    return sp;
  }
  // matrix time of one K step of a 256x256 tile on one CU, in us (dense
  // 4096 x 17408 x 5120 runs: MXFP8 2.0, MXFP4 2.6, NVFP4 on the FP16 matrix
  // cores 7.6)
  const double step_us = p.mode == kMXFP8 ? 2.0 : (p.mode == kMXFP4 ? 2.6 : 7.6);
  if (p.num_groups == 1 && tiles <= grid_full && tiles * 3 > grid_full && grid_full <= kSkMaxGrid) {
    // stream-K: K units of at least two steps, on scale-group boundaries.
    // Each workgroup then moves about 1 MB of FP32 partial tiles (stores and
    // loads of up to two slots of its own and of the tile's other pieces),
    // which measured 30 us over 256 workgroups whatever the format: taken
    // where the steps saved on the longest run are worth 40 us or more
    // (NVFP4 512 x 17408 x 5120: 141 -> 119 us; MXFP4 at the same shape
    // saves 8 steps, 21 us, and ran 42 -> 57 us).
    const bool gs = p.mode == kNVFP4 || p.ldsf % 16 == 0;
    const int64_t spg = !gs ? 1 : (p.mode == kMXFP8 ? 4 : (p.mode == kMXFP4 ? 2 : 1));
    const int64_t unit = spg < 2 ? 2 : spg;
    const int64_t upt = nk / unit;
    // the kernel's groups: grid_full / nx workgroups and at most
    // ceil(tiles / nx) tiles each (nx = 8 XCDs, or 1 below 8 CUs)
    const int64_t nx = grid_full >= 8 ? 8 : 1, per = grid_full / nx;
    const int64_t tpg = (tiles + nx - 1) / nx;
    const int64_t run = (tpg * upt + per - 1) / per;                   // units of the longest run
    const double saved_us = (double)(nk - run * unit) * step_us;
    if (nk % unit == 0 && upt >= 4 && run * 10 <= upt * 7 && saved_us >= 40.0) {
      sp.kind = kSplitStream;
      sp.grid = grid_full;
      sp.upt = (int32_t)upt;
      sp.unit = (int32_t)unit;
      sp.bytes = kWsHeader + 2 * (uint64_t)grid_full * BM * BN * 4;   // two partial slots per workgroup
      return sp;
    }
  }
  if (tiles * 2 <= cus && nk >= 8) {
    int64_t S = cus / tiles;
    if (S > nk / 4) S = nk / 4;
    if (S > 8) S = 8;
    // taken where the steps saved outweigh 1.5 times the partial planes'
    // HBM traffic (S planes written and read, the output written, at 5 TB/s):
    // MXFP4 512 x 12288 x 5120 (96 tiles, S = 2) saves 10 steps, 26 us,
    // against 23 us of traffic, and ran 40 us unsplit against 43 us split
    const double saved_us = (double)(nk - (nk + S - 1) / S) * step_us;
    const double traffic_us = (double)(S * 8 + 2) * (double)(p.m_rows * p.n) / 5.0e6;
    if (S >= 2 && saved_us >= 1.5 * traffic_us) {
      sp.kind = kSplitAll;
      sp.S = S;
      sp.bytes = kWsHeader + (uint64_t)(S * p.m_rows * p.n * 4);
    }
  }
  return sp;
}

namespace {

// The flag value of a stream-K call (its low word; a counter, so that calls
// in a row differ).  The flags are zero again when a call ends; a graph
// replay repeats its captured tag, which stays correct for that reason.
uint32_t next_sk_tag() {
  static std::atomic<uint32_t> tag{0x51u};
  return tag.fetch_add(1, std::memory_order_relaxed);
}

template <int FMT, bool GS>
hipError_t launch_tiled_cfg(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  const int smem = Lay<FMT, GS>::SMEM;
  // the dynamic-LDS attribute, once per device and instantiation (setting it
  // twice from racing threads is harmless)
  static std::atomic<bool> attr_set[64];
  const bool cached = dev.device >= 0 && dev.device < 64;
  if (!cached || !attr_set[dev.device].load(std::memory_order_acquire)) {
    const void* fns[] = {(const void*)mx_gemm_tiled<FMT, kEpiBf16, GS>, (const void*)mx_gemm_tiled<FMT, kEpiF16, GS>,
                         (const void*)mx_gemm_tiled<FMT, kEpiSplit, GS>,
                         (const void*)mx_gemm_tiled<FMT, kEpiBf16, GS, true>,
                         (const void*)mx_gemm_tiled<FMT, kEpiF16, GS, true>,
                         (const void*)mx_gemm_tiled<FMT, kEpiSplit, GS, true>,
                         (const void*)mx_gemm_tiled<FMT, kEpiStream, GS>};
    for (const void* fn : fns) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
      if (e != hipSuccess) return e;
    }
    if (cached) attr_set[dev.device].store(true, std::memory_order_release);
  }
  // Masked slots of at most BM rows: every weight tile is read by one m-tile
  // only, by every CU at once, so the weights stream from HBM and their loads
  // take the non-temporal policy (masked MXFP4 at E=64, K=7168, N=4096: 8-9 %
  // faster).  Measured against it elsewhere: dense MXFP4 4096x17408x5120,
  // whose weight tiles 16 m-tiles read, 12 % slower; dense 256x17408x5120
  // (one m-tile, but K-split over a part of the CUs) 21 % slower.
  const bool ntb = p.form == kMasked && p.slot_rows <= BM;
  auto go = [&](auto epi, int64_t grid, const GemmArgs& q) {
    constexpr int E = decltype(epi)::value;
    if (ntb)
      hipLaunchKernelGGL((mx_gemm_tiled<FMT, E, GS, true>), dim3((unsigned)grid), dim3(Cfg<FMT>::THREADS), smem, s, q);
    else
      hipLaunchKernelGGL((mx_gemm_tiled<FMT, E, GS, false>), dim3((unsigned)grid), dim3(Cfg<FMT>::THREADS), smem, s, q);
  };
  using EpiBf16 = std::integral_constant<int, kEpiBf16>;
  using EpiF16 = std::integral_constant<int, kEpiF16>;
  using EpiSplit = std::integral_constant<int, kEpiSplit>;
  const int64_t NT = (p.n + BN - 1) / BN;
  int64_t gm_upper;
  if (p.form == kContiguous) gm_upper = (p.m_rows + BM - 1) / BM + p.num_groups;
  else gm_upper = (int64_t)p.num_groups * ((p.slot_rows + BM - 1) / BM);
  const int64_t tiles = gm_upper * NT;
  const int cus = plan_cus(p, dev);
  const int64_t grid_full = cus >= 8 ? cus - cus % 8 : cus;
  // the split, if the plan has one and the caller's workspace holds it
  const SplitPlan sp = plan_split(p, dev);
  const bool split = sp.kind != kSplitNone && p.workspace != nullptr && p.workspace_bytes >= sp.bytes;
  float* const partial = split ? reinterpret_cast<float*>(static_cast<uint8_t*>(p.workspace) + kWsHeader) : nullptr;

  if (split && sp.kind == kSplitStream) {
    GemmArgs q = p;
    q.ksplit = 1;
    q.tile_limit = 0;
    q.partial = partial;
    q.sk_flags = static_cast<uint64_t*>(p.workspace);
    q.sk_upt = sp.upt;
    q.sk_unit = sp.unit;
    q.sk_tag = next_sk_tag();
    hipLaunchKernelGGL((mx_gemm_tiled<FMT, kEpiStream, GS>), dim3((unsigned)sp.grid), dim3(Cfg<FMT>::THREADS), smem,
                       s, q);
    return hipGetLastError();
  }

  if (split && sp.kind == kSplitTail) {
    // The last round's tiles -- a rectangle of whole n-tile columns of the
    // last block of m-tiles -- run after the others as a K-split sub-problem
    // (operand, scale, bias and output pointers offset to its corner; the
    // split reduce writes with the full output's row stride).
    const int64_t r0 = sp.r0, c0 = sp.c0;
    GemmArgs q2 = p;
    q2.a = p.a + r0 * p.lda;
    q2.sfa = p.sfa + r0 * p.ldsf;
    q2.b = p.b + c0 * p.lda;
    q2.sfb = p.sfb + c0 * p.ldsf;
    q2.out = p.out + r0 * p.n + c0;
    q2.bias = p.bias ? p.bias + c0 : nullptr;
    q2.m_rows = p.m_rows - r0;
    q2.slot_rows = q2.m_rows;
    q2.n = p.n - c0;
    q2.ldo = p.n;
    q2.ksplit = (int32_t)sp.S;
    q2.tile_limit = 0;
    q2.partial = partial;
    GemmArgs q1 = p;
    q1.ksplit = 1;
    q1.partial = nullptr;
    q1.tile_limit = (int32_t)(tiles - sp.rect_tiles);
    if (q1.out_f16) go(EpiF16{}, grid_full, q1);
    else go(EpiBf16{}, grid_full, q1);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
      int64_t g2 = sp.rect_tiles * sp.S;
      if (g2 > grid_full) g2 = grid_full;
      if (g2 >= 8) g2 -= g2 % 8;
      go(EpiSplit{}, g2, q2);
      e = hipGetLastError();
    }
    if (e == hipSuccess) {
      int64_t rgrid = (int64_t)cus * 4;
      if (q2.m_rows < rgrid) rgrid = q2.m_rows;
      hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)rgrid), dim3(256), 0, s, q2);
      e = hipGetLastError();
    }
    return e;
  }

  // K split of every tile (few tiles, long K)
  GemmArgs q = p;
  q.ksplit = 1;
  q.partial = nullptr;
  if (split && sp.kind == kSplitAll) {
    q.ksplit = (int32_t)sp.S;
    q.partial = partial;
  }
  int64_t grid = cus;
  if (tiles * q.ksplit < grid) grid = tiles * q.ksplit;
  if (grid >= 8) grid -= grid % 8;     // whole rounds over the 8 XCDs
  if (grid < 1) grid = 1;
  if (q.ksplit > 1) go(EpiSplit{}, grid, q);
  else if (q.out_f16) go(EpiF16{}, grid, q);
  else go(EpiBf16{}, grid, q);
  hipError_t e = hipGetLastError();
  if (q.ksplit > 1 && e == hipSuccess) {
    int64_t rgrid = (int64_t)cus * 4;
    if (p.m_rows < rgrid) rgrid = p.m_rows;
    hipLaunchKernelGGL(splitk_reduce, dim3((unsigned)rgrid), dim3(256), 0, s, q);
    e = hipGetLastError();
  }
  return e;
}

// The gate|up GEMM with the SwiGLU + re-quant epilogue: grouped-contiguous
// MXFP8, h / 128 n-tiles of 128 gate + 128 up weight rows each.
template <bool GS>
hipError_t launch_swiglu_cfg(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  const int smem = Lay<0, GS>::SMEM;
  static std::atomic<bool> attr_set[64];
  const bool cached = dev.device >= 0 && dev.device < 64;
  if (!cached || !attr_set[dev.device].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)mx_gemm_tiled<0, kEpiSwiglu, GS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)mx_gemm_tiled<0, kEpiSwiglu, GS, false, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    if (cached) attr_set[dev.device].store(true, std::memory_order_release);
  }
  const int64_t tiles = ((p.m_rows + BM - 1) / BM + p.num_groups) * (p.h / 128);
  const int cus = plan_cus(p, dev);
  int64_t grid = cus;
  if (tiles < grid) grid = tiles;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  GemmArgs q = p;
  q.ksplit = 1;
  q.partial = nullptr;
  q.tile_limit = 0;
  if (p.bias == nullptr)
    hipLaunchKernelGGL((mx_gemm_tiled<0, kEpiSwiglu, GS, false, true>), dim3((unsigned)grid), dim3(Cfg<0>::THREADS),
                       smem, s, q);
  else
    hipLaunchKernelGGL((mx_gemm_tiled<0, kEpiSwiglu, GS>), dim3((unsigned)grid), dim3(Cfg<0>::THREADS), smem, s, q);
  return hipGetLastError();
}

// The backward grouped GEMM with the dSwiGLU epilogue: grouped-contiguous,
// MXFP8 or MXFP4, 256-column n-tiles of R.
template <int FMT, bool GS>
hipError_t launch_dswiglu_cfg(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  const int smem = Lay<FMT, GS>::SMEM;
  static std::atomic<bool> attr_set[64];
  const bool cached = dev.device >= 0 && dev.device < 64;
  if (!cached || !attr_set[dev.device].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)mx_gemm_tiled<FMT, kEpiDswiglu, GS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)mx_gemm_tiled<FMT, kEpiDswigluQ, GS>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    if (cached) attr_set[dev.device].store(true, std::memory_order_release);
  }
  const int64_t tiles = ((p.m_rows + BM - 1) / BM + p.num_groups) * ((p.n + BN - 1) / BN);
  const int cus = plan_cus(p, dev);
  int64_t grid = cus;
  if (tiles < grid) grid = tiles;
  if (grid >= 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  GemmArgs q = p;
  q.ksplit = 1;
  q.partial = nullptr;
  q.tile_limit = 0;
  if (p.q_out != nullptr)
    hipLaunchKernelGGL((mx_gemm_tiled<FMT, kEpiDswigluQ, GS>), dim3((unsigned)grid), dim3(Cfg<FMT>::THREADS), smem,
                       s, q);
  else
    hipLaunchKernelGGL((mx_gemm_tiled<FMT, kEpiDswiglu, GS>), dim3((unsigned)grid), dim3(Cfg<FMT>::THREADS), smem,
                       s, q);
  return hipGetLastError();
}

}  // namespace

bool tiled_supported(const GemmArgs& p);

bool gemm_dswiglu_supported(const GemmArgs& p) {
  return (p.mode == kMXFP8 || p.mode == kMXFP4) && p.form == kContiguous && p.n % 32 == 0 &&
         p.n * 1024 < ((int64_t)1 << 31) && tiled_supported(p);
}

hipError_t launch_gemm_dswiglu(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  const bool gs = p.ldsf % 16 == 0;
  if (p.mode == kMXFP8) return gs ? launch_dswiglu_cfg<0, true>(s, p, dev) : launch_dswiglu_cfg<0, false>(s, p, dev);
  return gs ? launch_dswiglu_cfg<4, true>(s, p, dev) : launch_dswiglu_cfg<4, false>(s, p, dev);
}

bool gemm_swiglu_supported(const GemmArgs& p) {
  // the paired B loads reach h + 127 rows past a tile's first gate row with
  // 32-bit byte offsets
  return p.mode == kMXFP8 && p.form == kContiguous && p.h > 0 && p.h % 128 == 0 && p.n == 2 * p.h &&
         (p.h + 256) * p.lda < ((int64_t)1 << 31) && tiled_supported(p);
}

hipError_t launch_gemm_swiglu(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  return p.ldsf % 16 == 0 ? launch_swiglu_cfg<true>(s, p, dev) : launch_swiglu_cfg<false>(s, p, dev);
}

bool tiled_supported(const GemmArgs& p) {
  const int64_t step = p.mode == kMXFP8 ? 128 : 256;
  if (p.k % step != 0 || p.k < 2 * step) return false;   // at least two K steps
  if ((reinterpret_cast<uintptr_t>(p.sfa) | reinterpret_cast<uintptr_t>(p.sfb)) & 3) return false;
  if (p.lda * 256 >= (int64_t)1 << 31) return false;
  if (p.n * 256 * 2 > 0x7FFFFFFFLL) return false;   // 32-bit output offsets below the drop marker
  return true;
}

hipError_t launch_gemm_tiled(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  // grouped scale loads where a row's scale bytes are a multiple of 16 (NVFP4:
  // always, K % 256 == 0 gives K / 16 % 16 == 0)
  const bool gs = p.ldsf % 16 == 0;
  if (p.mode == kNVFP4) return launch_tiled_cfg<kNV, true>(s, p, dev);
  if (p.mode == kMXFP8) return gs ? launch_tiled_cfg<0, true>(s, p, dev) : launch_tiled_cfg<0, false>(s, p, dev);
  return gs ? launch_tiled_cfg<4, true>(s, p, dev) : launch_tiled_cfg<4, false>(s, p, dev);
}

}  // namespace hq
