// LDS-tiled, double-buffered scaled-MFMA GEMM for the MX modes (MXFP8 and
// MXFP4) -- the large-M tier of the flashrt/fp4-gemm page's M-tiered dispatch
// and the grouped MoE GEMMs of the HALOps "GEMM" page (group_contiguous_gemm,
// group_masked_gemm, batch_gemm sections).
//
// Structure (gfx950):
//   * 256 threads = 4 waves in a 2 x 2 grid; a block tile is BM x BN output
//     elements, a wave tile (BM/2) x (BN/2) built from 16 x 16 fragments of
//     V_MFMA_SCALE_F32_16X16X128_F8F6F4 (weights as src0, activations as
//     src1, FP32 accumulation, E8M0 scales per 32-element block).
//   * One K step moves 128 bytes of every row: 128 FP8 elements (one MFMA
//     step) or 256 FP4 elements (two MFMA steps).  A lane reads 16-byte
//     chunks q and q + 4 of its fragment row in both cases, so the LDS read
//     pattern is format independent.
//   * Global -> LDS with 16-byte direct-to-LDS loads (no register staging).
//     A wave's load writes 1 KB of LDS = 8 rows; lane j fetches the chunk that
//     belongs at LDS slot j, so the XOR swizzle (chunk ^ ((row ^ row>>3) & 7))
//     costs nothing and fragment reads are bank-conflict free.
//   * Two LDS stages: the loads of step k+1 are in flight while step k is
//     multiplied.
//   * Persistent grid (one workgroup per compute unit).  Tiles are ordered so
//     that the 32 consecutive tiles that one XCD (one L2) runs side by side
//     cover 4 row tiles x 8 column tiles: A and B tiles are shared through
//     the L2 instead of being fetched 32 times.
// Requirements (checked by the dispatcher): K % 128 == 0 (FP8) or
// K % 256 == 0 (FP4), scale rows 4-byte aligned.
#include "gemm_common.hpp"

namespace hq {
namespace {

constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) const void* lds_cptr_t;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// 32-bit LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_cptr_t)p;
}

// Direct-to-LDS loads: every lane fetches `size` bytes from sbase + voff and
// the wave's 64 results land contiguously at LDS address m0 (lane j at
// m0 + j * size).  Issued as inline assembly so that the compiler inserts no
// alias waits of its own: the kernel orders these writes explicitly (wait for
// the vector-memory counter, then a workgroup barrier, before a stage is read;
// a barrier after the last read of a stage before it is refilled).  m0 is set
// inside each statement; nothing else in the kernel uses it.
// A pointer the compiler cannot prove uniform (it came through LDS), made
// uniform explicitly; the value is the same in every lane.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  uint64_t v = (uint64_t)(uintptr_t)p;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

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

template <int FMT, int BM, int BN>
struct TiledCfg {
  static constexpr int SB = FMT == 0 ? 4 : 8;          // scale bytes per row per K step
  static constexpr int PLANES = SB / 4;                  // dword planes of scales
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BN * 128;
  static constexpr int SA_BYTES = BM * SB;
  static constexpr int SBB_BYTES = BN * SB;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SBB_BYTES;
  static constexpr int FM = BM / 32;                     // fragments per wave (rows)
  static constexpr int FN = BN / 32;                     // fragments per wave (cols)
  static constexpr int A_LOADS = BM / 32;                // 16-byte loads per thread per K step
  static constexpr int B_LOADS = BN / 32;
};

template <int FMT, int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void mx_gemm_tiled(GemmArgs p) {
  using C = TiledCfg<FMT, BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileTable tt;

  const int G = p.num_groups;
  const int NT = (int)((p.n + BN - 1) / BN);
  const int mt_per = p.form == kUniform ? (int)((p.slot_rows + BM - 1) / BM) : 0;
  int total_gm;
  if (p.form == kUniform) total_gm = G * mt_per;
  else total_gm = build_tile_table(p, BM, tt);
  const int total = total_gm * NT;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int q = lane >> 4, r16 = lane & 15;
  const int wm = w >> 1, wn = w & 1;
  const int nk = (int)(p.lda / 128);

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs,
  // so workgroup b runs on XCD b % 8.  Rounds of gridDim tiles; inside a
  // round XCD x owns a contiguous run of tiles.
  const int nxcd = gridDim.x >= 8 ? 8 : 1;
  const int per_xcd = gridDim.x / nxcd;
  const int slot = (blockIdx.x % nxcd) * per_xcd + blockIdx.x / nxcd;
  const bool slot_ok = (int)blockIdx.x < per_xcd * nxcd;

  for (int round = 0; slot_ok; ++round) {
    const int t = round * (per_xcd * nxcd) + slot;
    if (t >= total) break;
    // tile t -> (group m-tile gm, n tile nt): blocks of 4 m-tiles x all n-tiles,
    // walked n-major inside the block so 32 consecutive tiles = 4 m x 8 n.
    const int blk = t / (4 * NT);
    const int rem = t - blk * 4 * NT;
    const int mrem = total_gm - blk * 4;
    const int mb = mrem < 4 ? mrem : 4;
    const int nt = rem / mb;
    const int gm = blk * 4 + (rem - nt * mb);

    int g;
    int64_t row0, row_end;
    if (p.form == kUniform) {
      g = gm / mt_per;
      int mt = gm - g * mt_per;
      int64_t gs = (int64_t)g * p.slot_rows;
      row0 = gs + (int64_t)mt * BM;
      row_end = row0 + BM < gs + p.slot_rows ? row0 + BM : gs + p.slot_rows;
    } else {
      g = tile_group(tt, G, gm);
      int mt = gm - (g > 0 ? tt.mt_prefix[g - 1] : 0);
      row0 = (int64_t)tt.start[g] + (int64_t)mt * BM;
      int64_t ge = (int64_t)tt.start[g] + tt.count[g];
      row_end = row0 + BM < ge ? row0 + BM : ge;
    }
    const int64_t n0 = (int64_t)nt * BN;

    // ---- per-thread sources for the direct-to-LDS loads, as 32-bit offsets
    // from uniform tile bases.  Load i of wave w fills LDS rows
    // [(i*4 + w) * 8, +8); lane j -> row + j/8, physical chunk j % 8, logical
    // chunk (j % 8) ^ swz(row).  Rows past the tile end re-read a valid row.
    const uint8_t* a_base = uniform_ptr(p.a + row0 * p.lda);
    const uint8_t* b_base = uniform_ptr(p.b + (int64_t)g * p.b_stride + n0 * p.lda);
    uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
    const int64_t a_rows = row_end - row0;
    const int64_t b_rows = p.n - n0 < BN ? p.n - n0 : BN;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      int row = (i * 4 + w) * 8 + (lane >> 3);
      int c = (lane & 7) ^ swz(row);
      int rr = row < a_rows ? row : (int)a_rows - 1;
      a_off[i] = (uint32_t)(rr * p.lda + c * 16);
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      int row = (i * 4 + w) * 8 + (lane >> 3);
      int c = (lane & 7) ^ swz(row);
      int rr = row < b_rows ? row : (int)b_rows - 1;
      b_off[i] = (uint32_t)(rr * p.lda + c * 16);
    }
    // scales: dword plane h of row r sits at plane h * rows + r; wave w loads
    // rows [64w, 64w + 64) of each plane (waves past the tile skip).
    const uint8_t* sa_base = uniform_ptr(p.sfa + row0 * p.ldsf);
    const uint8_t* sb_base = uniform_ptr(p.sfb + (int64_t)g * p.sfb_stride + n0 * p.ldsf);
    uint32_t sa_off, sb_off;
    {
      int row = w * 64 + lane;
      int ra = row < a_rows ? row : (int)a_rows - 1;
      int rb = row < b_rows ? row : (int)b_rows - 1;
      sa_off = (uint32_t)(ra * p.ldsf);
      sb_off = (uint32_t)(rb * p.ldsf);
    }

    // sbase operands must be wave-uniform: every address above is built from
    // uniform values, and the LDS bases go through readfirstlane.
    auto issue = [&](int ks, const uint8_t* st) {
      const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(st) + w * 1024);
      const uint32_t lb = la + C::A_BYTES;
      const uint32_t lsa = __builtin_amdgcn_readfirstlane(lds_addr(st) + C::A_BYTES + C::B_BYTES + w * 256);
      const uint32_t lsb = lsa + C::SA_BYTES;
      const uint8_t* ak = a_base + ks * 128;
      const uint8_t* bk = b_base + ks * 128;
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) dma16(ak, a_off[i], la + i * 4096);
#pragma unroll
      for (int i = 0; i < C::B_LOADS; ++i) dma16(bk, b_off[i], lb + i * 4096);
      const uint8_t* sak = sa_base + ks * C::SB;
      const uint8_t* sbk = sb_base + ks * C::SB;
#pragma unroll
      for (int h = 0; h < C::PLANES; ++h) {
        if (w * 64 < BM) dma4(sak + 4 * h, sa_off, lsa + h * BM * 4);
        if (w * 64 < BN) dma4(sbk + 4 * h, sb_off, lsb + h * BN * 4);
      }
    };

    v4f acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    issue(0, smem);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int ks = 0; ks < nk; ++ks) {
      const uint8_t* cur = smem + (ks & 1) * C::STAGE;
      // 1. the next K step's loads go out first and fly during this step
      if (ks + 1 < nk) issue(ks + 1, smem + ((ks + 1) & 1) * C::STAGE);
      const uint8_t* la = cur;
      const uint8_t* lb = cur + C::A_BYTES;
      const uint8_t* lsa = cur + C::A_BYTES + C::B_BYTES;
      const uint8_t* lsb = lsa + C::SA_BYTES;

      // 2. the wave's B fragments (weights, src0) stay in registers
      uint4 blo[C::FN], bhi[C::FN];
      uint32_t bsc[C::FN][C::PLANES];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        int row = wn * (BN / 2) + j * 16 + r16;
        const uint8_t* rp = lb + row * 128;
        int s = swz(row);
        blo[j] = lds_read16(rp + ((q ^ s) << 4));
        bhi[j] = lds_read16(rp + (((q + 4) ^ s) << 4));
#pragma unroll
        for (int h = 0; h < C::PLANES; ++h)
          bsc[j][h] = (*reinterpret_cast<const uint32_t*>(lsb + h * BN * 4 + row * 4) >> (8 * q)) & 0xFFu;
      }
      // 3. A fragments stream through, each against every B fragment
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        int row = wm * (BM / 2) + i * 16 + r16;
        const uint8_t* rp = la + row * 128;
        int s = swz(row);
        uint4 alo = lds_read16(rp + ((q ^ s) << 4));
        uint4 ahi = lds_read16(rp + (((q + 4) ^ s) << 4));
        uint32_t asc[C::PLANES];
#pragma unroll
        for (int h = 0; h < C::PLANES; ++h)
          asc[h] = (*reinterpret_cast<const uint32_t*>(lsa + h * BM * 4 + row * 4) >> (8 * q)) & 0xFFu;
        if (FMT == 0) {
          v8i af = v8i{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            v8i bf = v8i{(int)blo[j].x, (int)blo[j].y, (int)blo[j].z, (int)blo[j].w,
                         (int)bhi[j].x, (int)bhi[j].y, (int)bhi[j].z, (int)bhi[j].w};
            acc[i][j] = mfma_scaled<0>(bf, af, acc[i][j], (int)bsc[j][0], (int)asc[0]);
          }
        } else {
          v8i af0 = v8i{(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, 0, 0, 0, 0};
          v8i af1 = v8i{(int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w, 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            v8i bf0 = v8i{(int)blo[j].x, (int)blo[j].y, (int)blo[j].z, (int)blo[j].w, 0, 0, 0, 0};
            v8i bf1 = v8i{(int)bhi[j].x, (int)bhi[j].y, (int)bhi[j].z, (int)bhi[j].w, 0, 0, 0, 0};
            acc[i][j] = mfma_scaled<4>(bf0, af0, acc[i][j], (int)bsc[j][0], (int)asc[0]);
            acc[i][j] = mfma_scaled<4>(bf1, af1, acc[i][j], (int)bsc[j][C::PLANES - 1], (int)asc[C::PLANES - 1]);
          }
        }
      }
      // 4. stage hand-over: keep every instruction of this step above the wait
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    // ---- epilogue: lane holds out[m = row][n = 4q + r] of each fragment
    const uint16_t* bias = p.bias ? p.bias + (int64_t)g * p.n : nullptr;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int64_t m = row0 + wm * (BM / 2) + i * 16 + r16;
      if (m < row_end) {
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int64_t n = n0 + wn * (BN / 2) + j * 16 + 4 * q;
          if (n < p.n) store_bf16x4(p.out + m * p.n + n, acc[i][j], bias ? bias + n : nullptr);
        }
      }
    }
  }
}

template <int FMT, int BM, int BN>
hipError_t launch_tiled_cfg(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  using C = TiledCfg<FMT, BM, BN>;
  const size_t smem = 2 * (size_t)C::STAGE;
  static bool attr_set = false;   // per process; the attribute is per function
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)mx_gemm_tiled<FMT, BM, BN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
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
  hipLaunchKernelGGL((mx_gemm_tiled<FMT, BM, BN>), dim3((unsigned)grid), dim3(kThreads), smem, s, p);
  return hipGetLastError();
}

}  // namespace

bool tiled_supported(const GemmArgs& p) {
  if (p.mode == kNVFP4) return false;
  const int64_t step = p.mode == kMXFP8 ? 128 : 256;
  if (p.k % step != 0) return false;
  if ((reinterpret_cast<uintptr_t>(p.sfa) | reinterpret_cast<uintptr_t>(p.sfb)) & 3) return false;
  if (p.lda * 256 >= (int64_t)1 << 31) return false;
  return true;
}

hipError_t launch_gemm_tiled(hipStream_t s, const GemmArgs& p, const DeviceInfo& dev) {
  if (p.mode == kMXFP8) return launch_tiled_cfg<0, 256, 256>(s, p, dev);
  return launch_tiled_cfg<4, 256, 256>(s, p, dev);
}

}  // namespace hq
