// Grouped expert GEMMs over the dispatched slots, on MFMA.
//
// Method: the SwiGLU expert f(x) = (SiLU(x̄ΓW^gate) ⊙ x̄ΓW^up) W^down
// ("ACE: Adaptive Calibration-Free Expert Skipping for MoE-based LLMs",
// picx.dev summary page, Theoretical Foundation), applied to each kept slot
// and scaled by its router gate.
//
// Work unit ("tile"): one expert, up to BM = 16*RB of its sorted slot rows,
// and NW*16*NGW of its weight rows.  Each wave owns NGW 16-row weight groups:
// for gate/up the gate rows and the up rows of the same 8*NGW intermediate
// units, so SiLU(gate)*up is formed in registers; for down NGW adjacent
// groups of 16 output columns.  The contraction runs in chunks of CK k-steps
// (one 16-byte lane load each, 64*CK bytes of a row):
//   - weight fragments are loaded straight from HBM into registers in MFMA
//     operand layout (each weight byte is read once per tile), one chunk
//     ahead of the MFMAs;
//   - the slot rows (gathered token rows of h, or act rows) are staged
//     through LDS and shared by all waves of the tile: through registers
//     into two LDS buffers, or (128-row tiles) by direct-to-LDS buffer loads
//     into a ring of three buffers, two chunks ahead of the MFMAs.
// In the 128-row tier a tile of at most 32 slot rows (an expert with
// few kept slots, or the ragged last m-tile of a larger one) multiplies only
// its own row blocks and spends the freed accumulator registers on a deeper
// weight ring; its outputs have the same bits as in a full tile.
// Every workgroup derives the tile list from expert_offsets (experts with no
// kept slot produce no tile, so their weights are never read) and takes the
// tile of its index.
#include "kernels.h"
#include "topk.h"

namespace ace {

namespace {

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef ACE_GROUPED_RB
#define ACE_GROUPED_RB 4      // 16-row blocks of slot rows per grouped tile
#endif
#ifndef ACE_GROUPED_STAGES
#define ACE_GROUPED_STAGES 2  // depth of the weight register ring (grouped tiles)
#endif
#ifndef ACE_WAVES_PER_EU
#define ACE_WAVES_PER_EU 3    // occupancy target given to the register allocator (4 to 7 row blocks;
                              // up to 3 row blocks fit 128 VGPRs with no spill and take 4)
#endif
#ifndef ACE_BIG_RB
#define ACE_BIG_RB 8          // 16-row blocks per tile for batches with >= ACE_BIG_SLOTS slots per expert
#endif
#ifndef ACE_BIG_NW
#define ACE_BIG_NW 4          // waves per tile of that tier
#endif
#ifndef ACE_BIG_NGW
#define ACE_BIG_NGW 4         // 16-row weight groups per wave of that tier (4 MFMAs per staged A fragment)
#endif
#ifndef ACE_BIG_CK
#define ACE_BIG_CK 2          // k-steps per chunk of that tier (keeps its weight ring within 64 VGPRs)
#endif
#ifndef ACE_BIG_STAGES
#define ACE_BIG_STAGES 2      // weight register ring depth of the big tier
#endif
#ifndef ACE_BIG_WPE
#define ACE_BIG_WPE 0         // occupancy target of the big tier (0: from the tile height)
#endif
#ifndef ACE_BIG_XB
#define ACE_BIG_XB 3          // LDS buffers of the big tier's direct-to-LDS row staging (0: staged through registers)
#endif
#ifndef ACE_BIG_AF
#define ACE_BIG_AF 2          // MFMA operand fragments per inline-assembly LDS read group (one-ring staging)
#endif
#ifndef ACE_BIG_CCR
#define ACE_BIG_CCR 1         // big gate/up tier: compiler-issued LDS reads from three separate arrays
                              // (0: inline-assembly read groups from one ring, as the down projection)
#endif
#ifndef ACE_LIGHT_RB
#define ACE_LIGHT_RB 2        // 128-row tier: tiles of at most 16*ACE_LIGHT_RB rows take the light
                              // path (only their row blocks' MFMAs, a deeper weight ring); 0: off
#endif
#ifndef ACE_LIGHT_STAGES
#define ACE_LIGHT_STAGES 3    // weight register ring depth of the light path (chunks)
#endif
#ifndef ACE_LIGHT_STAGES_DOWN
#define ACE_LIGHT_STAGES_DOWN 3  // the same for the down projection's light path (0: off)
#endif
#ifndef ACE_BIG_SLOTS
#define ACE_BIG_SLOTS 256     // routed slots per expert (on average) from which the big tier is used
#endif
#ifndef ACE_SMALL_NGW_GATEUP
#define ACE_SMALL_NGW_GATEUP 2  // weight groups per wave of the small gate/up tier
#endif
#ifndef ACE_SMALL_CK_GATEUP
#define ACE_SMALL_CK_GATEUP 4
#endif
#ifndef ACE_SMALL_NGW_DOWN
#define ACE_SMALL_NGW_DOWN 2    // weight groups per wave of the small down tier
#endif
#ifndef ACE_SMALL_CK_DOWN
#define ACE_SMALL_CK_DOWN 4
#endif
#ifndef ACE_MID_NGW
#define ACE_MID_NGW 4         // weight groups per wave of the 64-row tier
#endif
#ifndef ACE_MID_DOWN_WPE
#define ACE_MID_DOWN_WPE 2    // occupancy target of the 64-row tier's down projection (2 waves per SIMD: no spill)
#endif
#ifndef ACE_MID_CK
#define ACE_MID_CK 2          // k-steps per chunk of the 64-row tier
#endif
#ifndef ACE_SMALL_RB_GATEUP
#define ACE_SMALL_RB_GATEUP 3 // 16-row blocks per gate/up tile for moderate batches (<= 64 slots per expert)
#endif
#ifndef ACE_SMALL_RB_DOWN
#define ACE_SMALL_RB_DOWN 2   // the same for the down projection
#endif
#ifndef ACE_GATEUP_NW
#define ACE_GATEUP_NW 4       // waves per grouped gate/up tile (16 intermediate units each)
#endif
#ifndef ACE_DOWN_NW
#define ACE_DOWN_NW 4         // waves per grouped down tile (32 output columns each)
#endif
#ifndef ACE_XCD_COLUMNS
#define ACE_XCD_COLUMNS 1     // (expert, n-block) columns dealt round-robin over the XCDs: 0 never,
                              // 1 for the down projection (measured faster there), 2 for both kinds
#endif
#ifndef ACE_BIG_XCD_COLUMNS
#define ACE_BIG_XCD_COLUMNS 0 // the same for the 128-row tier (measured faster with contiguous parts)
#endif
#ifndef ACE_LDS_PITCH
#define ACE_LDS_PITCH 272     // padded LDS row pitch of the staged slot rows
#endif

constexpr int NXCD = 8;          // XCDs of an MI355X; only tile placement depends on it

// Whether tiles of RB row blocks and kind KIND deal their columns over the
// XCDs (else: the expert-major tile list in contiguous per-XCD parts).
template <int RB, int KIND>
constexpr bool columns_dealt() {
  constexpr int mode = RB >= ACE_BIG_RB ? ACE_BIG_XCD_COLUMNS : ACE_XCD_COLUMNS;
  return mode == 2 || (mode == 1 && KIND == 1);
}
constexpr int EMAX_EXP = 256;    // largest expert count
constexpr int LDS_PITCH = ACE_LDS_PITCH;

// Tile list of the dispatched slots (wave 0 writes it to LDS): expert e has
// ceil(n_e / BM) m-tiles; s_pref = exclusive prefix of those counts over the
// experts (s_pref[E] = total), s_off = expert_offsets.
template <int BM>
__device__ __forceinline__ void build_tile_list(const ExpertArgs& a, int32_t* s_pref, int32_t* s_off,
                                                int32_t* s_mte = nullptr, int mte_cap = 0) {
  if (wave_id() != 0) return;
  const int l = lane_id(), E = a.E;
  int cnt[4], loc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l * 4 + j;
    int c = 0;
    if (e < E) {
      const int o0 = a.offsets[e], o1 = a.offsets[e + 1];
      s_off[e] = o0;
      c = (o1 - o0 + BM - 1) / BM;
    }
    cnt[j] = c;
    loc += c;
  }
  const int inc = wave_incl_scan(loc);
  int run = inc - loc;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l * 4 + j;
    if (e < E) s_pref[e] = run;
    // optional m-tile table: the expert of each m-tile (entries past mte_cap dropped)
    if (s_mte != nullptr)
      for (int m = run; m < min(run + cnt[j], mte_cap); ++m) s_mte[m] = e;
    run += cnt[j];
  }
  if (l == 63) s_pref[E] = inc;
  if (l == 0) s_off[E] = a.offsets[E];
}

// Tile g of the expert-major list (expert, then n-block, then the expert's
// m-tiles): its expert, n-block, first sorted row and row count.
__device__ __forceinline__ void find_tile(int g, int nb_count, int BM, int E, const int32_t* s_pref,
                                          const int32_t* s_off, int& e, int& nb, int& row0, int& rows) {
  // expert e owns tiles [nb_count*s_pref[e], nb_count*s_pref[e+1])
  int lo = 0, hi = E;  // invariant: nb_count*s_pref[lo] <= g < nb_count*s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (nb_count * s_pref[mid] <= g) lo = mid; else hi = mid;
  }
  e = lo;
  const int mt_e = s_pref[e + 1] - s_pref[e];
  const int local = g - nb_count * s_pref[e];
  nb = local / mt_e;
  const int mtl = local - nb * mt_e;
  row0 = s_off[e] + mtl * BM;
  rows = min(BM, s_off[e + 1] - row0);
}

// Column-dealt tile list for one XCD.  A column is one (expert, n-block) pair
// with all of the expert's m-tiles; column c = e*nbc + nb goes to XCD c % 8,
// so a heavily loaded expert's columns spread over every XCD while each
// column's m-tiles (which reuse its weights) stay on one XCD's L2.  Wave 0
// writes s_pref[e] = exclusive prefix over experts of this XCD's tiles of
// expert e (its columns on the XCD times its m-tiles); s_off = expert_offsets.
template <int BM>
__device__ __forceinline__ int xcd_cols(int e, int x, int nbc) {
  const int r0 = (x - (e * nbc) % NXCD + NXCD) % NXCD;  // first n-block of expert e on XCD x
  return r0 < nbc ? (nbc - 1 - r0) / NXCD + 1 : 0;
}

template <int BM>
__device__ __forceinline__ void build_xcd_tile_list(const ExpertArgs& a, int x, int nbc, int32_t* s_pref,
                                                    int32_t* s_off) {
  if (wave_id() != 0) return;
  const int l = lane_id(), E = a.E;
  int cnt[4], loc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l * 4 + j;
    int c = 0;
    if (e < E) {
      const int o0 = a.offsets[e], o1 = a.offsets[e + 1];
      s_off[e] = o0;
      c = (o1 - o0 + BM - 1) / BM * xcd_cols<BM>(e, x, nbc);
    }
    cnt[j] = c;
    loc += c;
  }
  const int inc = wave_incl_scan(loc);
  int run = inc - loc;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l * 4 + j;
    if (e < E) s_pref[e] = run;
    run += cnt[j];
  }
  if (l == 63) s_pref[E] = inc;
  if (l == 0) s_off[E] = a.offsets[E];
}

// The j-th tile of XCD x's list: expert, n-block, first sorted row, row count.
template <int BM>
__device__ __forceinline__ void find_xcd_tile(int j, int x, int nbc, int E, const int32_t* s_pref,
                                              const int32_t* s_off, int& e, int& nb, int& row0, int& rows) {
  int lo = 0, hi = E;  // invariant: s_pref[lo] <= j < s_pref[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_pref[mid] <= j) lo = mid; else hi = mid;
  }
  e = lo;
  const int mt_e = (s_off[e + 1] - s_off[e] + BM - 1) / BM;
  const int local = j - s_pref[e];
  const int ck = local / mt_e, mtl = local - ck * mt_e;
  nb = (x - (e * nbc) % NXCD + NXCD) % NXCD + NXCD * ck;
  row0 = s_off[e] + mtl * BM;
  rows = min(BM, s_off[e + 1] - row0);
}

// s_waitcnt on the vector memory counter alone: vmcnt = N (6 bits: 3:0 and
// 15:14), expcnt and lgkmcnt at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier that orders LDS only: this wave's LDS operations
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for the
// vector memory loads in flight (__syncthreads' fence waits for every
// direct-to-LDS load, also those of later chunks); the caller waits for the
// direct-to-LDS loads the next chunk needs before calling it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct-to-LDS staging of one chunk by one wave: its DPW 1 KB blocks at
// dst + j*NW KB from per-lane byte offsets src[j] + soff.
template <int DPW, int NW>
__device__ __forceinline__ void stage_rows(__amdgpu_buffer_rsrc_t r, uint8_t* dst, const int* src,
                                           int soff) {
#pragma unroll
  for (int j = 0; j < DPW; ++j) buf_ld16_lds(r, dst + j * NW * 1024, src[j], soff);
}
// 16-byte LDS read issued by the compiler (it inserts the counter waits)
__device__ __forceinline__ u32x4 lds_rd16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Compile-time loop: f(integral_constant<int, i>) for i = 0 .. N-1.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// LDS reads of MFMA operands staged by direct-to-LDS loads.  The compiler
// cannot tell which LDS buffer a direct-to-LDS load writes, so before any LDS
// read it issued itself it waits for every such load in flight (vmcnt(0)),
// which would drain the staging ring each chunk.  These reads are issued from
// inline assembly instead, each group waiting for its own data (lgkmcnt(0))
// before the block ends; the caller has waited (vmcnt) for the loads that
// filled the buffer and passed a barrier.  NR reads of 16 bytes at byte
// addresses addr + OFF + i*STRIDE of LDS.
template <int NR, int OFF, int STRIDE>
__device__ __forceinline__ void lds_read_group(uint32_t addr, u32x4 (&v)[NR]) {
  static_assert(NR == 1 || NR == 2 || NR == 4, "1, 2 or 4 reads per group");
  static_assert(OFF >= 0 && OFF + (NR - 1) * STRIDE < 65536, "16-bit LDS offsets");
  if constexpr (NR == 1) {
    asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v[0]) : "v"(addr), "i"(OFF));
  } else if constexpr (NR == 2) {
    asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1])
                 : "v"(addr), "i"(OFF), "i"(OFF + STRIDE));
  } else {
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(addr), "i"(OFF), "i"(OFF + STRIDE), "i"(OFF + 2 * STRIDE), "i"(OFF + 3 * STRIDE));
  }
}

// WPE: occupancy target (waves per SIMD) given to the register allocator; 0
// picks it from the tile height.  XB > 0: the slot rows are staged with
// direct-to-LDS loads into XB buffers instead of through registers.
template <typename T, int RB, int NW, int KIND, int STAGES, int NGW = 2, int CK = 4, int WPE = 0, int XB = 0>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : (RB <= 3 ? 4 : (RB >= 16 ? 1 : (RB >= 8 ? 2 : ACE_WAVES_PER_EU))))))
void expert_gemm_kernel(ExpertArgs a) {
  static_assert(NGW % 2 == 0 && (CK == 2 || CK == 4), "weight groups per wave: even; k-steps per chunk: 2 or 4");
  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;      // k values per k-step
  constexpr int KC = CK * KS;      // k values per chunk
  constexpr int ROWBC = CK * 64;   // bytes of one staged row per chunk
  constexpr int PITCH = CK == 4 ? LDS_PITCH : ROWBC + 16;  // padded LDS row pitch (no bank conflicts)
  constexpr int BM = 16 * RB;
  constexpr int NTHR = NW * 64;
  constexpr int UNITS = BM * (ROWBC / 16);  // 16-byte units of one staged chunk
  constexpr int UPT = (UNITS + NTHR - 1) / NTHR;
  // output columns per wave and per tile: gate/up, NGW/2 groups of 16
  // intermediate units (their gate and their up rows); down, NGW groups of
  // 16 output columns
  constexpr int COLS_W = (KIND == 0) ? 8 * NGW : 16 * NGW;
  constexpr int ROWS_PER_WG = NW * COLS_W;
  // direct-to-LDS staging (XB > 0): XB buffers of unpadded 128-byte rows
  constexpr bool DMA = XB > 0;
  static_assert(!DMA || (CK == 2 && XB >= 3 && BM % (8 * NW) == 0),
                "direct-to-LDS staging: 2 k-steps per chunk, 3+ buffers, whole 1 KB blocks per wave");
  constexpr int NXB = DMA ? XB : 2;
  constexpr int XBYTES = DMA ? BM * ROWBC : BM * PITCH;
  constexpr bool CCR = DMA && ACE_BIG_CCR && KIND == 0;
  static_assert(!CCR || (XB == 3 && STAGES == 2), "compiler-issued reads: three buffers, two weight stages");
  // Light path of the direct-to-LDS tier: a tile with at most LBM slot rows
  // (an expert with few kept slots, or the last m-tile of a larger one)
  // multiplies only its LRB row blocks, so its time goes to the weight
  // stream; the registers the other row blocks' accumulators would hold
  // carry a deeper weight ring instead (LS chunks, LS - 1 in flight).
  constexpr int LRB = ACE_LIGHT_RB > 0 ? ACE_LIGHT_RB : 1;
  constexpr int LS = KIND == 0 ? ACE_LIGHT_STAGES : ACE_LIGHT_STAGES_DOWN;
  constexpr bool LIGHT = DMA && XB == 3 && (CCR || KIND == 1) && ACE_LIGHT_RB > 0 && LRB < RB && LS >= 2;
  constexpr int LBM = 16 * (LIGHT ? LRB : 1);
  static_assert(!LIGHT || (LBM % (8 * NW) == 0 && LS >= 2 && LS <= 6), "light path: whole 1 KB row blocks per wave");

  __shared__ __attribute__((aligned(16))) uint8_t s_x[CCR ? 1 : NXB][CCR ? 16 : XBYTES];
  // the three row buffers of the compiler-read staging (both paths of a tile)
  __shared__ __attribute__((aligned(16))) uint8_t s_r0[CCR ? XBYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_r1[CCR ? XBYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_r2[CCR ? XBYTES : 16];
  auto rbuf = [&](auto b) -> uint8_t* {
    if constexpr (int(b) == 0) return s_r0;
    else if constexpr (int(b) == 1) return s_r1;
    else return s_r2;
  };
  __shared__ int32_t s_pref[257];
  __shared__ int32_t s_off[257];

  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int q = l >> 4, r16 = l & 15;
  const int E = a.E, K = a.K, N = a.N;
  const int nch = K / KC;
  const int nb_count = N / ROWS_PER_WG;

  constexpr bool COLS = columns_dealt<RB, KIND>();
  const int xcd = int(blockIdx.x % NXCD);
  if (COLS)
    build_xcd_tile_list<BM>(a, xcd, nb_count, s_pref, s_off);
  else
    build_tile_list<BM>(a, s_pref, s_off);
  __syncthreads();

  const int ntiles = COLS ? s_pref[E] : s_pref[E] * nb_count;  // this XCD's / all tiles

  // Tile placement: workgroup id i runs on XCD i % NXCD (round-robin
  // dispatch) and takes the (i / NXCD)-th tile of that XCD's list.  With
  // column dealing (the down projection of the 32- to 64-row tiers by
  // default) an XCD's list holds every 8th (expert, n-block) column, each
  // column's m-tiles consecutive, so every XCD streams a share of every
  // expert and a column's weights are reused from one L2.  Otherwise (gate/up;
  // both kinds on the 128-row tiles) the expert-major list is cut into NXCD
  // contiguous parts, so that an expert's tiles share its weights and slot
  // rows on one XCD.  One
  // tile per workgroup; the hardware dispatcher refills a compute unit as soon
  // as one of its tiles finishes, which balances uneven per-CU bandwidth.
  const int per_xcd = COLS ? ntiles : (ntiles + NXCD - 1) / NXCD;
  for (int wg = blockIdx.x; wg < NXCD * per_xcd; wg += gridDim.x) {
    int e, nb, row0, rows;
    if (COLS) {
      find_xcd_tile<BM>(wg / NXCD, xcd, nb_count, E, s_pref, s_off, e, nb, row0, rows);
    } else {
      const int g = (wg % NXCD) * per_xcd + wg / NXCD;
      if (g >= ntiles) continue;
      find_tile(g, nb_count, BM, E, s_pref, s_off, e, nb, row0, rows);
    }
    const int nrb = (rows + 15) >> 4;

    // Weights are read with buffer loads: the expert's matrix base lives in a
    // scalar resource descriptor, the lane part of the address is one 32-bit
    // register and the k-step part a scalar offset.  k-step j of group g is at
    // byte wv + ws[g] + j * wstep.  Linear layout: row n0 + l%16, k offset
    // (l/16)*EPL.  Packed layout: fragment j of the group is one contiguous
    // 1 KB block in lane order.  Both 16-row groups of a wave are uniform.
    const int col0 = __builtin_amdgcn_readfirstlane(nb * ROWS_PER_WG + w * COLS_W);
    // weight group g: gate/up, g < NGW/2 the gate rows of units col0 + 16g
    // and g >= NGW/2 the up rows of the same units; down, the rows of output
    // columns col0 + 16g
    int n0[NGW];
#pragma unroll
    for (int g = 0; g < NGW; ++g) n0[g] = (KIND == 0) ? col0 + 16 * (g % (NGW / 2)) : col0 + 16 * g;
    const int64_t ebytes = int64_t(N) * K * int(sizeof(T));  // one expert's matrix
    const char* wm0 = reinterpret_cast<const char*>(a.W0) + int64_t(e) * ebytes;
    const char* wm1 = reinterpret_cast<const char*>((KIND == 0) ? a.W1 : a.W0) + int64_t(e) * ebytes;
    const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(wm0, uint32_t(ebytes));
    const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(wm1, uint32_t(ebytes));
    int wv, ws[NGW], wstep;
    if (a.packed) {
      const int ksteps = K / KS;
      wv = l * 16;
#pragma unroll
      for (int g = 0; g < NGW; ++g) ws[g] = (n0[g] / 16) * ksteps * 1024;
      wstep = 1024;
    } else {
      wv = (r16 * K + q * EPL) * int(sizeof(T));
#pragma unroll
      for (int g = 0; g < NGW; ++g) ws[g] = n0[g] * K * int(sizeof(T));
      wstep = KS * int(sizeof(T));
    }

    // weight chunks ride a register ring of STAGES chunks: while chunk c is
    // multiplied, the next STAGES-1 chunks are in flight.  The first chunks'
    // loads go out before the slot rows' sources are read (they depend only
    // on the tile), so the tile's start pays one memory latency, not two.
    u32x4 wA[NGW][CK], wB[NGW][CK], wC[NGW][CK];
    auto load_w = [&](u32x4 (&dst)[NGW][CK], int c) {
#pragma unroll
      for (int s = 0; s < CK; ++s)
#pragma unroll
        for (int g = 0; g < NGW; ++g)
          dst[g][s] = buf_ld16((KIND == 0 && g >= NGW / 2) ? wr1 : wr0, wv, ws[g] + (c * CK + s) * wstep);
    };
    if constexpr (LIGHT) {
      if (rows <= LBM) {
        // Same staging and operand layout as the full tile below, over LBM
        // rows: a chunk's rows go into three LDS buffers by direct-to-LDS
        // loads, each wave its own 1 KB blocks; gate/up reads the operands
        // from its three arrays by compiler-issued loads one fragment ahead,
        // down from its one-array ring by inline-assembly groups.  Each step
        // stages rows two chunks ahead and then loads weights LS - 1 chunks
        // ahead; MFMA chains run in the same k order as the full tile's, so a
        // row's outputs have the same bits.
        constexpr int LDPW = LBM / 8 / NW;  // 1 KB row blocks per wave and chunk
        constexpr int NWLL = NGW * CK;      // weight loads per wave and chunk
        u32x4 ring[LS][NGW][CK];
        static_for<LS - 1>([&](auto i) { load_w(ring[int(i)], min(int(i), nch - 1)); });
        f32x4 lacc[LRB][NGW];
#pragma unroll
        for (int rb = 0; rb < LRB; ++rb)
#pragma unroll
          for (int g = 0; g < NGW; ++g) lacc[rb][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        const __amdgpu_buffer_rsrc_t lxs = make_rsrc(a.A, uint32_t(int64_t(a.A_rows) * K * int(sizeof(T))));
        int ldsrc[LDPW];
#pragma unroll
        for (int j = 0; j < LDPW; ++j) {
          const int blk = j * NW + w;
          const int r = 8 * blk + (l >> 3);
          const int seg = (l & 7) ^ (l >> 3) ^ (blk & 1);
          const int rr = min(r, rows - 1);
          ldsrc[j] = ((KIND == 0) ? a.sorted_token[row0 + rr] : row0 + rr) * K * int(sizeof(T)) + seg * 16;
        }
        const int lsw = (r16 & 7) ^ (r16 >> 3);
        const int lrd[2] = {r16 * ROWBC + ((q ^ lsw) << 4), r16 * ROWBC + ((q ^ lsw ^ 4) << 4)};
        // the three row buffers: gate/up, the separate arrays read by the
        // compiler; down, the one-array ring read by inline-assembly groups
        auto lbuf = [&](auto b) -> uint8_t* {
          if constexpr (KIND == 0) return rbuf(b);
          else return s_x[int(b)];
        };
        const uint32_t lds_ring = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)(&s_x[0][0])));
        stage_rows<LDPW, NW>(lxs, lbuf(std::integral_constant<int, 0>{}) + w * 1024, ldsrc, 0);
        stage_rows<LDPW, NW>(lxs, lbuf(std::integral_constant<int, 1>{}) + w * 1024, ldsrc,
                             min(1, nch - 1) * KC * int(sizeof(T)));
        wait_vmcnt<LDPW>();
        lds_barrier();
        // step c: rows of chunk c + 2 into array (c + 2) % 3, weights of
        // chunk c + LS - 1 into ring slot (c - 1) % LS (read by step c - 1),
        // then the MFMAs of chunk c from array c % 3 and ring slot c % LS
        auto lstep = [&](auto B, auto RI, int c) {
          stage_rows<LDPW, NW>(lxs, lbuf(std::integral_constant<int, (int(B) + 2) % 3>{}) + w * 1024, ldsrc,
                               min(c + 2, nch - 1) * KC * int(sizeof(T)));
          load_w(ring[(int(RI) + LS - 1) % LS], min(c + LS - 1, nch - 1));
          __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
          if constexpr (KIND == 0) {
            const uint8_t* xb = lbuf(B);
            constexpr int NF = CK * LRB;  // operand fragments of the chunk, k-step major
            u32x4 af[2];
            af[0] = lds_rd16(xb + lrd[0]);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            static_for<NF>([&](auto f) {
              constexpr int s = int(f) / LRB, rb = int(f) % LRB;
              if constexpr (int(f) + 1 < NF)
                af[(int(f) + 1) & 1] = lds_rd16(xb + ((int(f) + 1) % LRB) * 16 * ROWBC + lrd[(int(f) + 1) / LRB]);
#pragma unroll
              for (int g = 0; g < NGW; ++g)
                lacc[rb][g] = mma_step<T>(af[int(f) & 1], ring[int(RI)][g][s], lacc[rb][g]);
              if constexpr (int(f) + 1 < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, NGW, 0);
            });
          } else {
            const uint32_t xb = lds_ring + uint32_t(int(B)) * XBYTES;
            static_for<CK>([&](auto s) {
              u32x4 af[LRB];
              lds_read_group<LRB, 0, 16 * ROWBC>(xb + uint32_t(lrd[int(s)]), af);
#pragma unroll
              for (int f = 0; f < LRB; ++f)
#pragma unroll
                for (int g = 0; g < NGW; ++g) lacc[f][g] = mma_step<T>(af[f], ring[int(RI)][g][int(s)], lacc[f][g]);
            });
          }
          // chunk c + 1's rows have landed once at most the loads issued
          // after them are outstanding: step c's alone at c = 0 (chunk 1
          // was staged by the prologue), else also step c - 1's weights
          if (c == 0)
            wait_vmcnt<NWLL + LDPW>();
          else
            wait_vmcnt<2 * NWLL + LDPW>();
          lds_barrier();
        };
        constexpr int LU = LS % 3 == 0 ? LS : 3 * LS;  // steps until array and ring slot repeat
        for (int c = 0; c < nch; c += LU)
          static_for<LU>([&](auto u) {
            if (c + int(u) < nch)
              lstep(std::integral_constant<int, int(u) % 3>{}, std::integral_constant<int, int(u) % LS>{}, c + int(u));
          });
        // the row offsets are formed here, not hoisted out of the tile loop
        // (where they would take registers for its whole length)
        int q4 = 4 * q;
        asm volatile("" : "+v"(q4));
#pragma unroll
        for (int rb = 0; rb < LRB; ++rb) {
          if (rb < nrb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = rb * 16 + q4 + j;
              if (r < rows) {
                const int64_t p = row0 + r;
                if constexpr (KIND == 0) {
#pragma unroll
                  for (int g = 0; g < NGW / 2; ++g) {
                    const float v = silu(lacc[rb][g][j]) * lacc[rb][g + NGW / 2][j];
                    reinterpret_cast<T*>(a.out)[p * N + col0 + 16 * g + r16] = St<T>::from_f32(v);
                  }
                } else {
                  const float gt = a.sorted_gate[p];
                  T* o = reinterpret_cast<T*>(a.out) + p * N + col0 + r16;
#pragma unroll
                  for (int g = 0; g < NGW; ++g) o[16 * g] = St<T>::from_f32(gt * lacc[rb][g][j]);
                }
              }
            }
          }
        }
        continue;
      }
    }
    load_w(wA, 0);
    if (STAGES == 3) load_w(wB, min(1, nch - 1));

    f32x4 acc[RB][NGW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int g = 0; g < NGW; ++g) acc[rb][g] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Rows past the tile's last slot row re-read that row: their MFMA output
    // rows are never stored (an output row depends only on its own input
    // row), and keeping every load unconditional keeps the loop body one block.
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.A, uint32_t(int64_t(a.A_rows) * K * int(sizeof(T))));
    if constexpr (DMA) {
      // Direct-to-LDS staging.  A 16-byte buffer load with the LDS flag puts
      // lane p's 16 bytes at a wave-uniform LDS base + 16p, so the chunk's
      // rows go from memory to LDS without passing through registers.  Row R
      // of a staged chunk is 128 unpadded bytes at R*128, its 16-byte segment
      // g in slot g ^ sw(R), sw(R) = (R & 7) ^ ((R >> 3) & 1): the 16 rows of
      // one MFMA operand read then fall in distinct bank groups (for 8- and
      // for 16-lane phases).  Load j of wave w fills the 1 KB block
      // b = j*NW + w (rows 8b..8b+7); lane p writes slot p%8 of row 8b + p/8
      // and so reads that row's segment (p%8) ^ sw.
      constexpr int DPW = BM / 8 / NW;  // 1 KB blocks per wave and chunk
      constexpr int NWL = NGW * CK;     // weight loads per wave and chunk
      int dsrc[DPW];
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        const int blk = j * NW + w;
        const int r = 8 * blk + (l >> 3);
        const int seg = (l & 7) ^ (l >> 3) ^ (blk & 1);
        const int rr = min(r, rows - 1);
        const int src_row = (KIND == 0) ? a.sorted_token[row0 + rr] : row0 + rr;
        dsrc[j] = src_row * K * int(sizeof(T)) + seg * 16;
      }
      // MFMA operand reads: row rb*16 + r16, k-step s of the chunk = segment 4s + q
      const int sw = (r16 & 7) ^ (r16 >> 3);
      const int rd[2] = {r16 * ROWBC + ((q ^ sw) << 4), r16 * ROWBC + ((q ^ sw ^ 4) << 4)};
      // Every step loads one chunk of weights and stages one chunk of rows
      // (past the last chunk: the last one again, a cache hit, into registers
      // or a buffer no later step of the tile reads), so the loads this wave
      // issues between two points are the same at every step.  The vector
      // memory counter completes in issue order, so "chunk c + 1 has landed"
      // is "at most the loads issued after it are outstanding".
      if constexpr (CCR) {
        // Three separate LDS arrays (each array's accesses carry their own
        // alias scope, so the compiler can tell a read of one array from a
        // load into another), the MFMA operands read by compiler-issued LDS
        // loads one fragment ahead of their MFMAs.  The compiler waits
        // before a chunk's first read for every direct-to-LDS load issued
        // before that step, so rows are staged one chunk ahead (chunk c + 2
        // is loaded during step c and waited for at the start of step c + 2,
        // with chunk c + 1's rows landing meanwhile).
        auto buf = [&](auto b) -> uint8_t* { return rbuf(b); };
        // step c: weights of chunk c + 1, rows of chunk c + 2 into array
        // (B + 2) % 3, the MFMAs of chunk c from array B = c % 3
        auto step = [&](auto B, u32x4 (&cur)[NGW][CK], u32x4 (&ahead)[NGW][CK], int c) {
          load_w(ahead, min(c + 1, nch - 1));
          stage_rows<DPW, NW>(xrs, buf(std::integral_constant<int, (int(B) + 2) % 3>{}) + w * 1024, dsrc,
                              min(c + 2, nch - 1) * KC * int(sizeof(T)));
          __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
          const uint8_t* xb = buf(B);
          constexpr int NF = CK * RB;  // operand fragments of the chunk, k-step major
          u32x4 af[2];
          af[0] = lds_rd16(xb + rd[0]);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // (groups: 0x100 LDS read, 0x008 MFMA)
          static_for<NF>([&](auto f) {
            constexpr int s = int(f) / RB, rb = int(f) % RB;
            if constexpr (int(f) + 1 < NF)
              af[(int(f) + 1) & 1] = lds_rd16(xb + ((int(f) + 1) % RB) * 16 * ROWBC + rd[(int(f) + 1) / RB]);
#pragma unroll
            for (int g = 0; g < NGW; ++g) acc[rb][g] = mma_step<T>(af[int(f) & 1], cur[g][s], acc[rb][g]);
            // in this order: the next fragment's read, then this fragment's MFMAs
            if constexpr (int(f) + 1 < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NGW, 0);
          });
          wait_vmcnt<NWL + DPW>();  // chunk c + 1's rows: only step c's loads may be outstanding
          lds_barrier();
        };
        stage_rows<DPW, NW>(xrs, s_r0 + w * 1024, dsrc, 0);
        stage_rows<DPW, NW>(xrs, s_r1 + w * 1024, dsrc, min(1, nch - 1) * KC * int(sizeof(T)));
        wait_vmcnt<DPW>();
        lds_barrier();
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using B2 = std::integral_constant<int, 2>;
        for (int c = 0; c < nch; c += 6) {  // array c % 3, weight ring c % 2
          step(B0{}, wA, wB, c);
          if (c + 1 < nch) step(B1{}, wB, wA, c + 1);
          if (c + 2 < nch) step(B2{}, wA, wB, c + 2);
          if (c + 3 < nch) step(B0{}, wB, wA, c + 3);
          if (c + 4 < nch) step(B1{}, wA, wB, c + 4);
          if (c + 5 < nch) step(B2{}, wB, wA, c + 5);
        }
      } else {
        // A ring of XB buffers in one array, rows staged XB - 1 chunks ahead
        // and the MFMA operands read by inline-assembly groups (the
        // compiler cannot tell which buffer of the array a direct-to-LDS
        // load writes, so before an LDS read of its own it would wait for
        // every such load in flight).  At the end of step c, chunk c + 1's
        // rows have landed once only the loads of the XB - 2 later steps
        // (weights, rows) are outstanding; for the first step of a 4-deep
        // ring, the prologue's last chunk stands in for one of them.
        constexpr int AF = ACE_BIG_AF;
        static_assert(RB % AF == 0, "row blocks per read group must divide the row blocks");
        const uint32_t lds_base = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)(&s_x[0][0])));
        // stage chunk c into the buffer of step slot (slot % XB)
        auto issue_x = [&](int c, int slot) {
          stage_rows<DPW, NW>(xrs, s_x[slot % XB] + w * 1024, dsrc, c * KC * int(sizeof(T)));
        };
        auto step = [&](u32x4 (&cur)[NGW][CK], u32x4 (&ahead)[NGW][CK], int c) {
          load_w(ahead, min(c + STAGES - 1, nch - 1));
          issue_x(min(c + XB - 1, nch - 1), c + XB - 1);
          __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
          const uint32_t xb = lds_base + uint32_t(c % XB) * XBYTES;
          static_for<CK>([&](auto s) {
            const uint32_t ad = xb + uint32_t(rd[int(s)]);
            static_for<RB / AF>([&](auto i) {
              u32x4 af[AF];
              lds_read_group<AF, int(i) * AF * 16 * ROWBC, 16 * ROWBC>(ad, af);
#pragma unroll
              for (int f = 0; f < AF; ++f)
#pragma unroll
                for (int g = 0; g < NGW; ++g)
                  acc[int(i) * AF + f][g] = mma_step<T>(af[f], cur[g][int(s)], acc[int(i) * AF + f][g]);
            });
          });
          if (XB >= 4 && c == 0)
            wait_vmcnt<(XB - 3) * DPW + NWL + DPW>();
          else
            wait_vmcnt<(XB - 2) * (NWL + DPW)>();
          lds_barrier();
        };
        for (int c = 0; c < XB - 1; ++c) issue_x(min(c, nch - 1), c);
        wait_vmcnt<(XB - 2) * DPW>();
        lds_barrier();
        if constexpr (STAGES == 3) {
          for (int c = 0; c < nch; c += 3) {
            step(wA, wC, c);
            if (c + 1 < nch) step(wB, wA, c + 1);
            if (c + 2 < nch) step(wC, wB, c + 2);
          }
        } else {
          for (int c = 0; c < nch; c += 2) {
            step(wA, wB, c);
            if (c + 1 < nch) step(wB, wA, c + 1);
          }
        }
      }
    } else {
      // staged-row sources of this thread's units (byte offsets into A)
      int xsrc[UPT];
      int xoff[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int unit = min(tid + u * NTHR, UNITS - 1);
        const int r = unit / (ROWBC / 16), seg = unit % (ROWBC / 16);
        xoff[u] = r * PITCH + seg * 16;
        const int rr = min(r, rows - 1);
        const int src_row = (KIND == 0) ? a.sorted_token[row0 + rr] : row0 + rr;
        xsrc[u] = src_row * K * int(sizeof(T)) + seg * 16;
      }

      u32x4 xr[UPT];
      auto load_x = [&](int c) {
        const int koff = c * KC * int(sizeof(T));
#pragma unroll
        for (int u = 0; u < UPT; ++u) xr[u] = buf_ld16(xrs, xsrc[u], koff);
      };
      auto store_x = [&](int buf) {
#pragma unroll
        for (int u = 0; u < UPT; ++u)
          if (UNITS % NTHR == 0 || tid + u * NTHR < UNITS) *reinterpret_cast<u32x4*>(&s_x[buf][xoff[u]]) = xr[u];
      };
      // One chunk.  Loads are issued X first, then weights: the X rows must land
      // before the barrier, and the in-order completion counter then lets the
      // weight loads of the later chunk stay in flight across it.  Every step
      // issues both (past the last chunk: the last chunk again, a cache hit):
      // with loads skipped on some paths the compiler's counter waits have to
      // hold on every path and so drain the loads just issued.
      auto step = [&](u32x4 (&cur)[NGW][CK], u32x4 (&ahead)[NGW][CK], int c) {
        load_x(min(c + 1, nch - 1));
        load_w(ahead, min(c + STAGES - 1, nch - 1));
        __builtin_amdgcn_sched_barrier(0);  // the loads go out before the MFMAs
        const int buf = c & 1;
#pragma unroll
        for (int s = 0; s < CK; ++s) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const u32x4 af = *reinterpret_cast<const u32x4*>(&s_x[buf][(rb * 16 + r16) * PITCH + s * 64 + q * 16]);
#pragma unroll
            for (int g = 0; g < NGW; ++g) acc[rb][g] = mma_step<T>(af, cur[g][s], acc[rb][g]);
          }
        }
        store_x(buf ^ 1);
        __syncthreads();
      };

      load_x(0);
      store_x(0);
      __syncthreads();
      if constexpr (STAGES == 3) {
        for (int c = 0; c < nch; c += 3) {
          step(wA, wC, c);
          if (c + 1 < nch) step(wB, wA, c + 1);
          if (c + 2 < nch) step(wC, wB, c + 2);
        }
      } else {
        for (int c = 0; c < nch; c += 2) {
          step(wA, wB, c);
          if (c + 1 < nch) step(wB, wA, c + 1);
        }
      }
    }

    // epilogue (row offsets formed here, not hoisted out of the tile loop)
    int q4 = 4 * q;
    asm volatile("" : "+v"(q4));
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb < nrb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = rb * 16 + q4 + j;
          if (r < rows) {
            const int64_t p = row0 + r;
            if (KIND == 0) {
#pragma unroll
              for (int g = 0; g < NGW / 2; ++g) {
                const float v = silu(acc[rb][g][j]) * acc[rb][g + NGW / 2][j];
                reinterpret_cast<T*>(a.out)[p * N + col0 + 16 * g + r16] = St<T>::from_f32(v);
              }
            } else {
              const float gt = a.sorted_gate[p];
              T* o = reinterpret_cast<T*>(a.out) + p * N + col0 + r16;
#pragma unroll
              for (int g = 0; g < NGW; ++g) o[16 * g] = St<T>::from_f32(gt * acc[rb][g][j]);
            }
          }
        }
      }
    }
  }
  // the last steps' direct-to-LDS loads land before the workgroup's LDS is released
  if constexpr (DMA) wait_vmcnt<0>();
}

// Small-batch ("stream") path: split-K inside the workgroup.  A tile is one
// expert, up to 16 of its slot rows and NGRP groups of 16 weight rows
// (gate/up: the 16 gate and the 16 up rows of the same intermediate units;
// down: 16*NGRP output columns).  Its SK_NW waves take interleaved k-steps
// (wave w: w, w+SK_NW, ...) and issue all weight and slot-row loads of up to
// SK_NBK k-steps at once, so that with few rows per expert the weight stream
// is limited by bandwidth, not by one wave's loads in flight.  The waves'
// partial sums meet in LDS and are added in wave order (deterministic, and
// the same bits for any NGRP), then SiLU(gate)*up or the gate scale is
// applied.  Slot rows are read straight from global memory (they are few and
// stay in L2).
constexpr int SK_NW = 8;
constexpr int SK_MT_CAP = 1024;  // m-tile table entries of the split-K kernel

template <typename T, int KIND, int SK_NBK, int NGRP>
__global__ __launch_bounds__(SK_NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void expert_splitk_kernel(ExpertArgs a) {
  static_assert(KIND == 1 || NGRP == 2, "gate/up tiles hold one gate and one up group");
  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;
  constexpr int BM = 16;
  constexpr int COLS = (KIND == 0) ? 16 : 16 * NGRP;  // output columns per tile
  __shared__ int32_t s_pref[257];
  __shared__ int32_t s_off[257];
  __shared__ int32_t s_mte[SK_MT_CAP];
  __shared__ float s_red[SK_NW][NGRP][16][17];

  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int q = l >> 4, r16 = l & 15;
  const int E = a.E, K = a.K, N = a.N;
  const int nb_count = N / COLS;
  const int nk = K / KS;
  const int nkw = w < nk ? (nk - 1 - w) / SK_NW + 1 : 0;  // this wave's k-steps

  build_tile_list<BM>(a, s_pref, s_off, s_mte, SK_MT_CAP);
  __syncthreads();
  // XCD x takes the x-th contiguous part of the tile list: m-tile-major
  // (m-tile, then n-block; expert and rows from the m-tile table) when the
  // table holds every m-tile, else expert-major with a binary search
  const int ntiles = s_pref[E] * nb_count;
  const bool table = s_pref[E] <= SK_MT_CAP;
  const int per_xcd = (ntiles + NXCD - 1) / NXCD;
  for (int wg = blockIdx.x; wg < NXCD * per_xcd; wg += gridDim.x) {
    const int g = (wg % NXCD) * per_xcd + wg / NXCD;
    if (g >= ntiles) continue;
    int e, nb, row0, rows;
    if (table) {
      const int mt = g / nb_count;
      nb = g - mt * nb_count;
      e = s_mte[mt];
      row0 = s_off[e] + BM * (mt - s_pref[e]);
      rows = min(BM, s_off[e + 1] - row0);
    } else {
      find_tile(g, nb_count, BM, E, s_pref, s_off, e, nb, row0, rows);
    }
    const int col0 = nb * COLS;
    const int64_t ebytes = int64_t(N) * K * int(sizeof(T));
    const char* wm0 = reinterpret_cast<const char*>(a.W0) + int64_t(e) * ebytes;
    const char* wm1 = reinterpret_cast<const char*>((KIND == 0) ? a.W1 : a.W0) + int64_t(e) * ebytes;
    const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(wm0, uint32_t(ebytes));
    const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(wm1, uint32_t(ebytes));
    // group gg: weight rows n0 = col0 (gate/up: both groups) or col0 + 16*gg (down)
    int wv, ws[NGRP], wstep;
    if (a.packed) {
      wv = l * 16;
#pragma unroll
      for (int gg = 0; gg < NGRP; ++gg) ws[gg] = ((KIND == 0 ? col0 : col0 + 16 * gg) / 16) * nk * 1024;
      wstep = 1024;
    } else {
      wv = (r16 * K + q * EPL) * int(sizeof(T));
#pragma unroll
      for (int gg = 0; gg < NGRP; ++gg) ws[gg] = (KIND == 0 ? col0 : col0 + 16 * gg) * K * int(sizeof(T));
      wstep = KS * int(sizeof(T));
    }
    f32x4 acc[NGRP];
#pragma unroll
    for (int gg = 0; gg < NGRP; ++gg) acc[gg] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nkw > 0) {
      // weight loads of the first batch go out before the slot row is known
      u32x4 wq[SK_NBK][NGRP], xa[SK_NBK];
      auto load_w = [&](int i0) {
#pragma unroll
        for (int b = 0; b < SK_NBK; ++b) {
          const int j = w + SK_NW * min(i0 + b, nkw - 1);
#pragma unroll
          for (int gg = 0; gg < NGRP; ++gg) wq[b][gg] = buf_ld16((KIND == 0 && gg == 1) ? wr1 : wr0, wv, ws[gg] + j * wstep);
        }
      };
      load_w(0);
      // slot row of this lane; lanes past the tile's last row get an offset
      // beyond the buffer, so their loads return zero without memory traffic
      const int rr = min(r16, rows - 1);
      const int src_row = (KIND == 0) ? a.sorted_token[row0 + rr] : row0 + rr;
      const uint32_t xbytes = uint32_t(int64_t(a.A_rows) * K * int(sizeof(T)));
      const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.A, xbytes);
      const int xv = r16 < rows ? (src_row * K + q * EPL) * int(sizeof(T)) : int(0x7FFFFFF0u);
      for (int i0 = 0; i0 < nkw; i0 += SK_NBK) {
        if (i0 > 0) load_w(i0);
#pragma unroll
        for (int b = 0; b < SK_NBK; ++b) {
          const int j = w + SK_NW * min(i0 + b, nkw - 1);
          xa[b] = buf_ld16(xrs, xv, j * KS * int(sizeof(T)));
        }
#pragma unroll
        for (int b = 0; b < SK_NBK; ++b) {
          if (i0 + b < nkw) {
#pragma unroll
            for (int gg = 0; gg < NGRP; ++gg) acc[gg] = mma_step<T>(xa[b], wq[b][gg], acc[gg]);
          }
        }
      }
    }
    // lane (q, r16) holds rows 4q..4q+3 of weight column r16 in each group
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int gg = 0; gg < NGRP; ++gg) s_red[w][gg][4 * q + j][r16] = acc[gg][j];
    __syncthreads();
    if (tid < 256) {
      const int row = tid >> 4, c = tid & 15;
      if (row < rows) {
        float v[NGRP];
#pragma unroll
        for (int gg = 0; gg < NGRP; ++gg) {
          v[gg] = s_red[0][gg][row][c];
#pragma unroll
          for (int ww = 1; ww < SK_NW; ++ww) v[gg] += s_red[ww][gg][row][c];
        }
        const int64_t p = row0 + row;
        if (KIND == 0) {
          reinterpret_cast<T*>(a.out)[p * N + col0 + c] = St<T>::from_f32(silu(v[0]) * v[1]);
        } else {
          const float gt = a.sorted_gate[p];
          T* o = reinterpret_cast<T*>(a.out) + p * N + col0 + c;
#pragma unroll
          for (int gg = 0; gg < NGRP; ++gg) o[16 * gg] = St<T>::from_f32(gt * v[gg]);
        }
      }
    }
    __syncthreads();  // s_red is reused by the next tile of this workgroup
  }
}

// The tile count is known only on the device; the grid covers the host-side
// bound but at most SK_WG_PER_CU workgroups per compute unit, which loop over
// the tiles (workgroups past the last tile exit after the tile-list prologue,
// so an uncapped worst-case grid would mostly pay that prologue).  k-steps
// per load batch: 8 for gate/up (K = H), 4 for down (K = I; fewer registers,
// more resident workgroups).  Down tiles are 32 output columns, or 64 from
// ACE_SK_DOWN_WIDE_SLOTS routed slots on, where the tiles outnumber the
// resident workgroups and twice the bytes in flight per workgroup pay.
#ifndef ACE_SK_WG_PER_CU
#define ACE_SK_WG_PER_CU 2      // grid cap per CU of the split-K kernel (measured best for decode)
#endif
#ifndef ACE_SK_DOWN_WIDE_SLOTS
#define ACE_SK_DOWN_WIDE_SLOTS 32
#endif
constexpr int SK_WG_PER_CU = ACE_SK_WG_PER_CU;

template <typename T, int KIND>
hipError_t launch_splitk(const ExpertArgs& a, int ntok, int k, int num_cu, hipStream_t s) {
  const int64_t slots = int64_t(ntok) * k;
  const bool wide = KIND == 1 && slots >= ACE_SK_DOWN_WIDE_SLOTS && a.N % 64 == 0;
  const int COLS = (KIND == 0) ? 16 : (wide ? 64 : 32);
  const int64_t mt_bound = (slots + 15) / 16 + std::min<int64_t>(a.E, slots);
  const int64_t tiles_bound = mt_bound * (a.N / COLS);
  const int64_t cap = int64_t(std::max(num_cu, 1)) * SK_WG_PER_CU;
  const int64_t grid = std::max<int64_t>(NXCD, (std::min(tiles_bound, cap) + NXCD - 1) / NXCD * NXCD);
  if (KIND == 0)
    hipLaunchKernelGGL((expert_splitk_kernel<T, 0, 8, 2>), dim3(unsigned(grid)), dim3(SK_NW * 64), 0, s, a);
  else if (wide)
    hipLaunchKernelGGL((expert_splitk_kernel<T, 1, 4, 4>), dim3(unsigned(grid)), dim3(SK_NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((expert_splitk_kernel<T, 1, 4, 2>), dim3(unsigned(grid)), dim3(SK_NW * 64), 0, s, a);
  return hipGetLastError();
}

// Fused small-batch gate/up (decode, T <= FUSED_TMAX): instead of reading
// the outputs of a separate top-k kernel and a dispatch kernel, every
// workgroup derives them from the router logits in LDS (a few hundred slots
// at most): wave w runs topk_slots for tokens w, w + 8, ... (the same code
// and bits as the routing kernel); kept (expert, token) pairs set bit t of a per-expert
// token mask, so expert e's count is the mask's popcount and slot (t, i)'s
// row is offset[e] + popcount(mask[e] below bit t) (token order, as in
// moe_dispatch); then the split-K tiles run as in expert_splitk_kernel.
// Workgroup 0 writes topk_idx, topk_gate, keep, expert_offsets,
// sorted_token, sorted_gate and slot_pos for the later kernels (down
// projection, combine) and the caller.  Saves two dependent launches.
// Two workgroups per CU (4 waves per SIMD) need at most 128 VGPRs.
template <typename T>
__global__ __launch_bounds__(SK_NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void expert_splitk_fused_kernel(FusedArgs f) {
  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;
  constexpr int BM = 16;
  constexpr int COLS = 16;
  constexpr int SK_NBK = 8;
  constexpr int MAXS = FUSED_TMAX * 16;
  static_assert(FUSED_TMAX <= 32, "an expert's tokens are a 32-bit mask");
  __shared__ float s_tg[EMAX_EXP], s_tr[EMAX_EXP];
  __shared__ double s_z[SK_NW][EMAX_EXP];
  __shared__ int32_t s_idx[MAXS];
  __shared__ float s_gate[MAXS];
  __shared__ uint8_t s_keep[MAXS];
  __shared__ uint32_t s_mask[EMAX_EXP];
  __shared__ int32_t s_pref[EMAX_EXP + 1];
  __shared__ int32_t s_off[EMAX_EXP + 1];
  __shared__ int32_t s_mte[MAXS / 16 + EMAX_EXP];  // expert of each m-tile (expert order)
  __shared__ int32_t s_tok[MAXS];
  __shared__ float s_red[SK_NW][2][16][17];
  const ExpertArgs& a = f.g;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int q = l >> 4, r16 = l & 15;
  const int E = a.E, K = a.K, N = a.N, k = f.k, Tn = f.T;
  const int nslots = Tn * k;
  const bool writer = blockIdx.x == 0;

  // 1. tables, masks, the first token's logits of each wave
  for (int e = tid; e < EMAX_EXP; e += SK_NW * 64) {
    const int ec = min(e, E - 1);
    s_tg[e] = f.a_gsp[ec];
    s_tr[e] = f.a_rcr[ec];
    s_mask[e] = 0u;
  }
  // lane l holds the logits of experts l*R .. l*R + R-1 (topk_slots' layout)
  const int R = topk_per_lane(E);
  float v[4];
  auto load_logits = [&](int t) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) v[rr] = rr < R ? f.logits[int64_t(min(t, Tn - 1)) * E + min(l * R + rr, E - 1)] : 0.f;
  };
  load_logits(w);
  __syncthreads();
  // 2. top-k, gates, skip decision: wave w for tokens w, w + SK_NW, ...
  {
    const TopkParams p{E, k, f.norm_topk, f.fusion, f.tau_gsp, f.tau_rcr};
    for (int t = w; t < Tn; t += SK_NW) {
      if (t > w) load_logits(t);
      int my_e;
      float g;
      bool kp;
      topk_slots(v, p, s_tg, s_tr, s_z[w], my_e, g, kp);
      if (l < k) {
        const int sidx = t * k + l;
        s_idx[sidx] = my_e;
        s_gate[sidx] = g;
        s_keep[sidx] = kp ? 1 : 0;
        if (kp) atomicOr(&s_mask[my_e], 1u << t);
        if (writer) {
          f.topk_idx[sidx] = my_e;
          f.topk_gate[sidx] = g;
          f.keep[sidx] = kp ? 1 : 0;
        }
      }
    }
  }
  __syncthreads();
  // 3. expert offsets and m-tile prefix: wave 0, lane l owns experts
  //    4l..4l+3; rows and m-tiles travel packed (rows << 16 | m-tiles, both
  //    at most FUSED_TMAX * 16 here) through one wave scan
  if (w == 0) {
    uint32_t pk[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * l + j;
      const int cnt = e < E ? __popc(s_mask[e]) : 0;
      pk[j] = (uint32_t(cnt) << 16) | uint32_t((cnt + BM - 1) / BM);
      tot += pk[j];
    }
    const uint32_t inc = uint32_t(wave_incl_scan(int(tot)));
    uint32_t run = inc - tot;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * l + j;
      if (e < E) {
        s_off[e] = int(run >> 16);
        s_pref[e] = int(run & 0xFFFFu);
        for (int m = 0; m < int(pk[j] & 0xFFFFu); ++m) s_mte[int(run & 0xFFFFu) + m] = e;
      }
      run += pk[j];
    }
    if (l == 63) {
      s_off[E] = int(inc >> 16);
      s_pref[E] = int(inc & 0xFFFFu);
    }
  }
  __syncthreads();
  // 4. rows of the kept slots (token order inside an expert)
  for (int sl = tid; sl < nslots; sl += SK_NW * 64) {
    const int t = sl / k;
    int row = -1;
    if (s_keep[sl]) {
      const int e = s_idx[sl];
      row = s_off[e] + __popc(s_mask[e] & ((1u << t) - 1u));
      s_tok[row] = t;
      if (writer) {
        f.sorted_token[row] = t;
        f.sorted_gate[row] = s_gate[sl];
      }
    }
    if (writer) f.slot_pos[sl] = row;
  }
  if (writer && tid <= E) f.offsets[tid] = s_off[tid];
  __syncthreads();

  // 5. split-K tiles over the LDS tile list, as in expert_splitk_kernel
  const int nb_count = N / COLS;
  const int nk = K / KS;
  const int nkw = w < nk ? (nk - 1 - w) / SK_NW + 1 : 0;
  const int ntiles = s_pref[E] * nb_count;
  // tile gi runs on XCD gi % 8 (the grid is a multiple of 8): dealt over the
  // XCDs, measured faster here than contiguous parts
  // tiles in m-tile-major order (m-tile, then n-block): the tile's expert
  // and rows come from the m-tile table in three LDS reads
  for (int gi = blockIdx.x; gi < ntiles; gi += gridDim.x) {
    const int mt = gi / nb_count, nb = gi - mt * nb_count;
    const int e = s_mte[mt];
    const int row0 = s_off[e] + BM * (mt - s_pref[e]);
    const int rows = min(BM, s_off[e + 1] - row0);
    const int col0 = nb * COLS;
    const int64_t ebytes = int64_t(N) * K * int(sizeof(T));
    const char* wm0 = reinterpret_cast<const char*>(a.W0) + int64_t(e) * ebytes;
    const char* wm1 = reinterpret_cast<const char*>(a.W1) + int64_t(e) * ebytes;
    const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(wm0, uint32_t(ebytes));
    const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(wm1, uint32_t(ebytes));
    int wv, ws, wstep;
    if (a.packed) {
      wv = l * 16;
      ws = (col0 / 16) * nk * 1024;
      wstep = 1024;
    } else {
      wv = (r16 * K + q * EPL) * int(sizeof(T));
      ws = col0 * K * int(sizeof(T));
      wstep = KS * int(sizeof(T));
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (nkw > 0) {
      u32x4 wa[SK_NBK], wb[SK_NBK], xa[SK_NBK];
      auto load_w = [&](int i0) {
#pragma unroll
        for (int b = 0; b < SK_NBK; ++b) {
          const int j = w + SK_NW * min(i0 + b, nkw - 1);
          wa[b] = buf_ld16(wr0, wv, ws + j * wstep);
          wb[b] = buf_ld16(wr1, wv, ws + j * wstep);
        }
      };
      load_w(0);
      const int src_row = s_tok[row0 + min(r16, rows - 1)];
      const uint32_t xbytes = uint32_t(int64_t(a.A_rows) * K * int(sizeof(T)));
      const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.A, xbytes);
      const int xv = r16 < rows ? (src_row * K + q * EPL) * int(sizeof(T)) : int(0x7FFFFFF0u);
      for (int i0 = 0; i0 < nkw; i0 += SK_NBK) {
        if (i0 > 0) load_w(i0);
#pragma unroll
        for (int b = 0; b < SK_NBK; ++b) {
          const int j = w + SK_NW * min(i0 + b, nkw - 1);
          xa[b] = buf_ld16(xrs, xv, j * KS * int(sizeof(T)));
        }
#pragma unroll
        for (int b = 0; b < SK_NBK; ++b) {
          if (i0 + b < nkw) {
            acc0 = mma_step<T>(xa[b], wa[b], acc0);
            acc1 = mma_step<T>(xa[b], wb[b], acc1);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s_red[w][0][4 * q + j][r16] = acc0[j];
      s_red[w][1][4 * q + j][r16] = acc1[j];
    }
    __syncthreads();
    if (tid < 256) {
      const int row = tid >> 4, c = tid & 15;
      if (row < rows) {
        float v0 = s_red[0][0][row][c], v1 = s_red[0][1][row][c];
#pragma unroll
        for (int ww = 1; ww < SK_NW; ++ww) {
          v0 += s_red[ww][0][row][c];
          v1 += s_red[ww][1][row][c];
        }
        const int64_t pr = row0 + row;
        reinterpret_cast<T*>(a.out)[pr * N + col0 + c] = St<T>::from_f32(silu(v0) * v1);
      }
    }
    __syncthreads();
  }
}

// Packed weight layout: [E][N/16][K/KS][64 lanes][16 bytes], where the
// 16-byte unit of lane l in fragment (e, n-group, k-step j) holds row
// n-group*16 + l%16, k values j*KS + (l/16)*EPL .. +EPL of the linear
// [E][N][K] matrix.  One thread copies one 16-byte unit.
template <typename T>
__global__ __launch_bounds__(256) void pack_weights_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t units,
                                                           int N, int K) {
  constexpr int EPL = St<T>::EPL;
  constexpr int KS = 4 * EPL;
  const int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (u >= units) return;
  const int l = int(u & 63);
  const int64_t frag = u >> 6;
  const int64_t ksteps = K / KS;
  const int64_t j = frag % ksteps;
  const int64_t rowgrp = frag / ksteps;  // e * (N/16) + n-group: rows of [E*N, K] in groups of 16
  const int64_t row = rowgrp * 16 + (l & 15);
  const int64_t k = j * KS + (l >> 4) * EPL;
  st16(dst + u * EPL, ld16(src + row * K + k));
}

template <typename T, int RB, int NW, int KIND, int STAGES, int NGW = 2, int CK = 4, int WPE = 0, int XB = 0>
hipError_t launch_one(const ExpertArgs& a, int ntok, int k, hipStream_t s) {
  constexpr int BM = 16 * RB;
  constexpr int ROWS_PER_WG = (KIND == 0) ? NW * 8 * NGW : NW * 16 * NGW;
  const int64_t slots = int64_t(ntok) * k;
  const int64_t mt_bound = (slots + BM - 1) / BM + std::min<int64_t>(a.E, slots);
  const int64_t nbc = a.N / ROWS_PER_WG;
  // the grid covers the largest possible tile count of any XCD (times NXCD);
  // workgroups past their XCD's actual count exit at once
  constexpr bool COLS = columns_dealt<RB, KIND>();
  const int64_t per_xcd_bound = COLS ? (nbc + NXCD - 1) / NXCD * mt_bound : (mt_bound * nbc + NXCD - 1) / NXCD;
  const int64_t grid = std::max<int64_t>(NXCD, std::min<int64_t>(per_xcd_bound * NXCD, int64_t(1) << 30));
  hipLaunchKernelGGL((expert_gemm_kernel<T, RB, NW, KIND, STAGES, NGW, CK, WPE, XB>), dim3(unsigned(grid)),
                     dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(int dtype, const void* src, void* dst, int E, int N, int K, hipStream_t s) {
  const int64_t bytes = int64_t(E) * N * K * (dtype == 1 ? 2 : 4);
  const int64_t units = bytes / 16;
  const dim3 grid(unsigned((units + 255) / 256)), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(pack_weights_kernel<bf16_t>, grid, block, 0, s, static_cast<const bf16_t*>(src),
                       static_cast<bf16_t*>(dst), units, N, K);
  else
    hipLaunchKernelGGL(pack_weights_kernel<float>, grid, block, 0, s, static_cast<const float*>(src),
                       static_cast<float*>(dst), units, N, K);
  return hipGetLastError();
}

#ifndef ACE_FUSED_WG_PER_CU
#define ACE_FUSED_WG_PER_CU 2   // grid cap of the fused kernel (about the resident count): its workgroups
                                // loop over the tiles, paying the routing prologue once (measured best)
#endif

hipError_t launch_fused_gateup(int dtype, const FusedArgs& a, int num_cu, hipStream_t s) {
  const int64_t slots = int64_t(a.T) * a.k;
  const int64_t mt_bound = (slots + 15) / 16 + std::min<int64_t>(a.g.E, slots);
  const int64_t tiles_bound = mt_bound * (a.g.N / 16);
  const int64_t cap = int64_t(std::max(num_cu, 1)) * ACE_FUSED_WG_PER_CU;
  const int64_t grid = std::max<int64_t>(NXCD, (std::min(tiles_bound, cap) + NXCD - 1) / NXCD * NXCD);
  if (dtype == 1)
    hipLaunchKernelGGL(expert_splitk_fused_kernel<bf16_t>, dim3(unsigned(grid)), dim3(SK_NW * 64), 0, s, a);
  else
    hipLaunchKernelGGL(expert_splitk_fused_kernel<float>, dim3(unsigned(grid)), dim3(SK_NW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_expert(int dtype, int kind, bool stream_path, const ExpertArgs& a, int T, int k, int num_cu,
                         hipStream_t s) {
  constexpr int G = ACE_GROUPED_RB, S = ACE_GROUPED_STAGES;
  // moderate batches (up to 64 routed slots per expert on average before
  // skipping): 48-row gate/up tiles and 32-row down tiles, each 4 per CU
  // (measured fastest at T = 1024, E = 128: 1536 gate/up and 2048+ down
  // tiles).  Large batches (at least ACE_BIG_SLOTS = 256 slots per expert):
  // 128-row tiles of 4 waves with 64 weight rows each, which cut the L2
  // traffic per MFMA when the GEMMs become compute-bound.  Between the two:
  // 64-row tiles.
  const bool small_rb = int64_t(T) * k <= int64_t(64) * a.E && G > 2;
  // (the big tile covers ACE_BIG_NW * 8 * ACE_BIG_NGW units or 16 * that many
  // output columns: N must be a multiple)
  const bool big_rb = int64_t(T) * k >= int64_t(ACE_BIG_SLOTS) * a.E &&
                      a.N % ((kind == 0 ? 8 : 16) * ACE_BIG_NW * ACE_BIG_NGW) == 0;
  if (dtype == 1) {
    if (stream_path)
      return kind == 0 ? launch_splitk<bf16_t, 0>(a, T, k, num_cu, s) : launch_splitk<bf16_t, 1>(a, T, k, num_cu, s);
    constexpr int NG = ACE_GATEUP_NW, ND = ACE_DOWN_NW;
    if (big_rb)
      return kind == 0
                 ? launch_one<bf16_t, ACE_BIG_RB, ACE_BIG_NW, 0, ACE_BIG_STAGES, ACE_BIG_NGW, ACE_BIG_CK, ACE_BIG_WPE,
                              ACE_BIG_XB>(a, T, k, s)
                 : launch_one<bf16_t, ACE_BIG_RB, ACE_BIG_NW, 1, ACE_BIG_STAGES, ACE_BIG_NGW, ACE_BIG_CK, ACE_BIG_WPE,
                              ACE_BIG_XB>(a, T, k, s);
    constexpr int SG = ACE_SMALL_NGW_GATEUP, SGC = ACE_SMALL_CK_GATEUP;
    constexpr int SD = ACE_SMALL_NGW_DOWN, SDC = ACE_SMALL_CK_DOWN;
    if (small_rb && a.N % ((kind == 0 ? 8 * NG * SG : 16 * ND * SD)) == 0)
      return kind == 0 ? launch_one<bf16_t, ACE_SMALL_RB_GATEUP, NG, 0, S, SG, SGC>(a, T, k, s)
                       : launch_one<bf16_t, ACE_SMALL_RB_DOWN, ND, 1, S, SD, SDC>(a, T, k, s);
    if (small_rb)
      return kind == 0 ? launch_one<bf16_t, ACE_SMALL_RB_GATEUP, NG, 0, S>(a, T, k, s)
                       : launch_one<bf16_t, ACE_SMALL_RB_DOWN, ND, 1, S>(a, T, k, s);
    constexpr int MID_NGW = ACE_MID_NGW, MID_CK = ACE_MID_CK;
    if (a.N % ((kind == 0 ? 8 : 16) * (kind == 0 ? NG : ND) * MID_NGW) == 0)
      return kind == 0 ? launch_one<bf16_t, G, NG, 0, S, MID_NGW, MID_CK>(a, T, k, s)
                       : launch_one<bf16_t, G, ND, 1, S, MID_NGW, MID_CK, ACE_MID_DOWN_WPE>(a, T, k, s);
    return kind == 0 ? launch_one<bf16_t, G, NG, 0, S>(a, T, k, s)
                     : launch_one<bf16_t, G, ND, 1, S>(a, T, k, s);
  }
  if (stream_path)
    return kind == 0 ? launch_splitk<float, 0>(a, T, k, num_cu, s) : launch_splitk<float, 1>(a, T, k, num_cu, s);
  // (float32 layers: two waves per SIMD, so the tile's registers fit without spilling)
  return kind == 0 ? launch_one<float, G, 4, 0, S, 2, 4, 2>(a, T, k, s)
                   : launch_one<float, G, 4, 1, S, 2, 4, 2>(a, T, k, s);
}

}  // namespace ace
