// Tiled 2:4 sparse GEMM for gfx950: K2 (2:4 sparse MFMA + LoRA, gemm_sparse32).
// The dense baseline K3 (gemm_dense32) is built the same way in
// k_gemm_dense.hip; the helpers both use are in lynx_tile.h.
//
// Layer (RT-Lynx page, 코드 예제, second formula; 방법론 "핵심 메커니즘" and
// "CUDA 커널 최적화": the 2:4 activation goes to the sparse unit, the LoRA
// output is generated and accumulated on chip inside the sparse GEMM):
//   Y = s * (X~ W^T) + T LA^T.
// The sparse product accumulates in fp32 registers; its rows are then scaled
// by s in place and the LoRA up-projection accumulates on top of them, on the
// same instruction, with T as stored.
//
// The kernel is persistent: one workgroup of 4 waves (2 x 2) per compute unit
// walks 256 x 256 (or 256 x 192) output tiles, each wave 128 x 128 (4 x 4
// accumulator tiles of 32 x 32, 256 fp32 per lane).  Operands move global ->
// LDS by buffer_load ... lds (no VGPR staging) into a ring of 3 LDS stages of
// 64 dense channels that runs on from one tile into the next: packed values
// 256 x 64 B, meta 256 x 8 B, W 256 x 128 B (50 KB, 1024 matrix-core cycles
// per wave).  The packed operand is stored in 16-row x 64-channel tiles, so a
// stage's A side is 16 contiguous 1 KB value tiles and 16 contiguous 128 B
// meta tiles.  The loads of a stage are waited for with an explicit vmcnt that
// leaves the later stages' loads in flight, then one s_barrier per stage;
// every load of the kernel is such an LDS-DMA, so the counts are exact.  Rows
// past M or N lie past the end of their buffer resource and read as zeros
// (they only reach outputs that are not stored).  LDS rows keep their 16-byte
// chunks XOR-swizzled by row so the fragment reads of 8 (and 16) consecutive
// lanes hit distinct banks.  Y is written through a buffer resource (32-bit
// offsets), straight from the accumulators for interior tiles, through an
// 8-row LDS transpose for edge tiles.
//
// Tile order: workgroups are handed to the 8 XCDs round-robin, so ids are
// remapped to give each XCD a contiguous range of tiles, and tiles are
// rasterized in groups of 8 tile-rows so the ~32 workgroups resident on one
// XCD share A rows and W rows in that XCD's L2.
#include <type_traits>

#include "lynx_tile.h"

namespace lynx {
namespace {

// K2's stage: 64 dense channels of a 256 x (64 NB) tile (NB = 4 or 3 column
// blocks of 32 per wave)
template <int NB>
struct Cfg {
    static_assert(NB == 3 || NB == 4, "tile widths 192 and 256");
    static constexpr int TILE_N = 64 * NB;               // tile columns
    static constexpr int BK = 64;                        // dense channels per stage
    static constexpr int A_ROW = 64;                     // LDS bytes per A row per stage
    static constexpr int B_ROW = 128;                    // LDS bytes per B row per stage
    static constexpr int A_BYTES = BM * A_ROW;
    static constexpr int META_BYTES = BM * 8;
    static constexpr int B_BYTES = TILE_N * B_ROW;
    static constexpr int STAGE = A_BYTES + META_BYTES + B_BYTES;
    static constexpr int NSTAGE = 3;
    static constexpr int A_DMA = A_BYTES / 1024 / 4;     // 1 KB DMA instructions per wave
    static constexpr int B_DMA = B_BYTES / 1024 / 4;
    static constexpr int M_DMA = META_BYTES / 256 / 4;   // 256 B (dword) DMA instructions
    static constexpr int DMA_PER_STAGE = A_DMA + B_DMA + M_DMA;
    static constexpr int SCALE_OFF = NSTAGE * STAGE;     // s of the tile's 256 rows
    static_assert(2 * DMA_PER_STAGE < 64, "vmcnt range");
};

// ---------------------------------------------------------------------------
// K2: Y = s * (X~ W^T) + T LA^T with v_smfmac_f32_32x32x32_bf16.
//
// Each wave's 128 x 128 is 4 x 4 accumulator tiles of 32 x 32 (16 fp32 each).
// A stage is two 32-channel sub-steps of 16 SMFMACs (32 cycles each).  The
// fragments of one sub-step take 52 VGPRs (A: 4 x (8 values + index word),
// B: 4 x 16 values), so two sets fit beside the accumulators and alternate by
// sub-step.  Every DMA and LDS read is issued between two SMFMACs (order pinned
// by sched_barrier), so the matrix core keeps issuing while they are queued.
//
// Lane l, r = l % 32, h = l / 32 (layouts pinned by the probe tests):
//   A = row r, dense channels [16h, 16h+16) of the 32-channel sub-step: 8 kept
//     values (chunk 2 sub + h of the 64-byte LDS row) + 16-bit index word;
//   B = column r, channels [8h, 8h+8) and [16+8h, 24+8h): chunks 4 sub + h and
//     4 sub + 2 + h of the 128-byte LDS row;
//   D = column r, rows 8 (e / 4) + 4 h + e % 4, e = 0..15.
// The LoRA up-projection runs on the same instruction (after the main loop).
// ---------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(NT, 1) void gemm_sparse32(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta,
    const float* __restrict__ scale, const uint16_t* __restrict__ T,
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ LA,
    uint16_t* __restrict__ Y, int M, int N, int K, int R) {
    using C = Cfg<NB>;
    constexpr int TN = C::TILE_N;   // tile columns
    constexpr int WC = 32 * NB;     // columns per wave
    // ring of 3 stages, the tile's s, and the epilogue's staging rows
    constexpr int kEpiOff = C::SCALE_OFF + BM * 4;
    constexpr int kEpiWave = 8 * 256;  // 8 rows x 128 columns bf16 per wave
    constexpr int kLds = kEpiOff + 4 * kEpiWave;
    static_assert(kLds <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, h = lane >> 5;
    const int wm = wave & 1, wn = wave >> 1;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + TN - 1) / TN;
    const int ntiles = tiles_m * tiles_n;

    // ---- DMA addressing ----------------------------------------------------
    // values: instruction j of wave w moves the 1 KB value tile of row block
    //   (m0/16 + w + 4j) into LDS rows 16 (w + 4j) .. +16 (64 B each);
    // meta (dword DMA, 256 B): the two 128 B tiles of row blocks 2 (w + 4j)
    //   and 2 (w + 4j) + 1 into LDS rows 32 (w + 4j) .. +32 (8 B each);
    // W (128-byte LDS rows): instruction j moves rows 8 (w + 4j) + l/8.
    // Lane l lands at LDS byte 16 l (4 l) of the instruction's 1 KB (256 B);
    // its source is the chunk the row's swizzle puts there.
    const uint32_t lds0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
    const int steps = K / 64;
    const int Mp = (M + 15) & ~15;
    const i32x4 rsA = make_rsrc(values, uint32_t(Mp) * uint32_t(K));
    const i32x4 rsB = make_rsrc(W, uint32_t(N) * uint32_t(2 * K));
    const i32x4 rsM = make_rsrc(meta, uint32_t(Mp) * uint32_t(K / 8));
    const i32x4 rsT = make_rsrc(T, uint32_t(M) * uint32_t(2 * R));
    const i32x4 rsL = make_rsrc(LA, uint32_t(N) * uint32_t(2 * R));
    const i32x4 rsS = make_rsrc(scale, uint32_t(M) * 4u);
    uint32_t voffA[C::A_DMA], voffB[C::B_DMA], voffM[C::M_DMA];
    auto set_tile_offsets = [&](int tm0, int tn0) {
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j) {
            const int blk = wave + 4 * j, row = lane >> 2, ph = lane & 3;
            voffA[j] = uint32_t(tm0 / 16 + blk) * uint32_t(steps) * 1024u + uint32_t(row * 64 + 16 * (ph ^ swz64(row)));
        }
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j) {
            const int row = 8 * (wave + 4 * j) + (lane >> 3), ph = lane & 7;
            voffB[j] = uint32_t(tn0 + row) * uint32_t(2 * K) + uint32_t(16 * (ph ^ swz128(row)));
        }
#pragma unroll
        for (int j = 0; j < C::M_DMA; ++j) {
            // rows 16..31 of each 32-row group (lanes 32..63) land with their
            // two dwords swapped, so a fragment's 32 rows read 32 banks
            const int blk = 2 * (wave + 4 * j) + (lane >> 5);
            voffM[j] = uint32_t(tm0 / 16 + blk) * uint32_t(steps) * 128u + uint32_t(4 * ((lane & 31) ^ (lane >> 5)));
        }
    };
    // one of the DMA instructions of a stage (4 value tiles, 2 meta, 2 NB W)
    auto dma_k = [&](int t, uint32_t slot_off, int k) {
        const uint32_t base = lds0 + slot_off;
        if (k < C::A_DMA) {
            dma16(base + 1024 * (wave + 4 * k), voffA[k], rsA, uint32_t(t) * 1024u);
        } else if (k < C::A_DMA + C::M_DMA) {
            const int j = k - C::A_DMA;
            dma4(base + C::A_BYTES + 256 * (wave + 4 * j), voffM[j], rsM, uint32_t(t) * 128u);
        } else {
            const int j = k - C::A_DMA - C::M_DMA;
            dma16(base + C::A_BYTES + C::META_BYTES + 1024 * (wave + 4 * j), voffB[j], rsB, uint32_t(t) * 128u);
        }
    };

    // ---- fragments ---------------------------------------------------------
    // Two fragment sets (one per 32-channel sub-step) alternate.  SMFMACs run
    // column-block-major, k = 4 b + a, and a set's 8 + 2 NB LDS reads are
    // issued in the order that consumes them: A0, B0, A1, A2, A3, B1, B2 (, B3).
    constexpr int kS = 4 * NB;          // SMFMACs per sub-step
    constexpr int kReads = 8 + 2 * NB;  // LDS reads per fragment set
    const int s64 = swz64(r), s128 = swz128(r);
    const int offA = (wm * 128 + r) * 64;      // + 32 a rows (a * 2048 bytes)
    const int offM = (wm * 128 + r) * 8;       // + a * 256
    const int offB = (wn * WC + r) * 128;      // + b * 4096
    struct Frags {
        bf16x8 v[4];
        int i[4];
        bf16x8 blo[NB], bhi[NB];
    };
    Frags fr[2];
    // read n (0 .. kReads-1) of a set, from the ring slot at byte offset soff
    auto read_n = [&](int soff, int sub, Frags& f, int n) {
        const char* As = smem + soff;
        const char* Bs = As + C::A_BYTES + C::META_BYTES;
        // n -> (A row block, values / index) or (B column block, low / high half)
        constexpr int kind[16] = {0, 1, 2, 3, 0, 1, 0, 1, 0, 1, 2, 3, 2, 3, 2, 3};
        constexpr int blk[16] = {0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 1, 1, 2, 2, 3, 3};
        const int x = blk[n];
        switch (kind[n]) {
            case 0:
                f.v[x] = lds_read<bf16x8>(As, offA + x * 2048 + 16 * ((2 * sub + h) ^ s64));
                break;
            case 1:
                f.i[x] = lds_read<uint16_t>(As + C::A_BYTES, offM + x * 256 + 2 * (2 * (sub ^ (r >> 4)) + h));
                break;
            case 2:
                f.blo[x] = lds_read<bf16x8>(Bs, offB + x * 4096 + 16 * ((4 * sub + h) ^ s128));
                break;
            default:
                f.bhi[x] = lds_read<bf16x8>(Bs, offB + x * 4096 + 16 * ((4 * sub + 2 + h) ^ s128));
                break;
        }
    };

    f32x16 acc[4][NB];
    auto mma = [&](const Frags& f, int k) {
        const int a = k & 3, b = k >> 2;
        const bf16x16 bv = __builtin_shufflevector(f.blo[b], f.bhi[b], 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                                   9, 10, 11, 12, 13, 14, 15);
        acc[a][b] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(f.v[a], bv, acc[a][b], f.i[a], 0, 0);
    };

    // Ring schedule.  Stage u's DMA instructions (14 at width 256, 12 at 192)
    // go out in two halves: the first half starts in stage u - 3's sub-step 1,
    // after the barrier that frees slot u % 3 (kPartA instructions; the other
    // kPartB of the first half, when the slots run short, join the second
    // half), and the second half goes out in stage u - 2's sub-step 0.  Per
    // stage t (set 0 holds sub-step 0's fragments):
    //   sub-step 0: SMFMACs on set 0; two reads of set 1 (same slot) after
    //     each of the first kR2, then the DMAs of stage t + 2 (kPartB + half),
    //     about one after each remaining SMFMAC;
    //   sub-step 1: one SMFMAC on set 1; wait for stage t + 1's loads and this
    //     wave's reads; barrier (slot t % 3 is free); the other SMFMACs, the
    //     first kR2 each followed by two reads of stage t + 1's set 0, the next
    //     kPartA by one DMA of stage t + 3's first half into slot t % 3.
    // Every memory instruction sits between two SMFMACs (sched_barrier), so
    // the matrix core keeps issuing while they are queued, and no SMFMAC slot
    // carries both fragment reads and DMAs: the LDS serves both, and keeping
    // them apart (with the barrier after the first SMFMAC of sub-step 1
    // rather than the fourth) took 7% off the cycles of an MLP-up launch.
    // The two stages after a tile's last one carry its LoRA operands through
    // the same slots: "stage" nk is the tile's 256 rows of T and "stage"
    // nk + 1 its 256 rows of LA, 8 DMA instructions each (128-byte rows; ranks
    // past R and rows past M or N read as zeros), so they arrive while the
    // last stages compute; stage nk also brings the tile's 256 values of s
    // (rows past M read as 0) into their own LDS table.  Every load of the
    // kernel is one of these DMA instructions, so all vmcnt waits are explicit
    // and count them exactly; loads complete in order, so a wait that leaves
    // the n loads issued after a stage in flight has that stage landed,
    // whatever the epilogue's stores in between are doing.  "Stage" nk + 2 is the next tile's stage 0: the
    // workgroup is persistent (tiles blockIdx.x, + gridDim.x, ...), and the
    // next tile's first loads are in flight during this tile's LoRA and
    // epilogue.
    constexpr int kHalf = C::DMA_PER_STAGE / 2;
    static_assert(C::DMA_PER_STAGE == 2 * kHalf && kHalf <= 8 && kHalf >= 5, "DMA split");
    constexpr int kLoraHalf = 4;  // T DMA instructions per half of the T stage
    constexpr int kLaHalf = NB;   // LA DMA instructions per half of the LA stage
    constexpr int kR2 = kReads / 2;  // SMFMAC slots with reads, per sub-step
    constexpr int kBar = 1;          // SMFMACs of sub-step 1 before its wait and barrier
    // first-half DMAs after sub-step 1's reads; the rest join the second half
    constexpr int kPartA = kS - kBar - kR2 < kHalf ? kS - kBar - kR2 : kHalf;
    constexpr int kPartB = kHalf - kPartA;
    static_assert(kPartA > 0 && kPartB >= 0 && kR2 + kBar <= kS, "stage slots");
    const int nk = K / 64;  // >= 2: the dispatcher sends K = 64 to the 64 x 64 kernel
    enum { kMain, kT, kLA, kNext0 };
    int m0 = 0, n0 = 0;
    // LoRA DMA instruction j (0..7) of wave w: LDS rows 8 (w + 4j) + l/8 of
    // the slot (128 B each), 16-byte chunk l % 8 in swizzled position
    auto dma_lora = [&](bool is_T, int soff, int j) {
        const int row = 8 * (wave + 4 * j) + (lane >> 3);
        const int c = (lane & 7) ^ swz128(row);
        const int base = is_T ? m0 : n0;
        const uint32_t voff = 8 * c < R ? uint32_t(base + row) * uint32_t(2 * R) + uint32_t(16 * c) : 0xFFFFFFF0u;
        dma16(lds0 + uint32_t(soff) + 1024 * (wave + 4 * j), voff, is_T ? rsT : rsL, 0);
    };
    // wave w's quarter of the tile's s: rows 64 w + l
    auto dma_scale = [&]() {
        dma4(lds0 + C::SCALE_OFF + 256 * wave, uint32_t(m0 + 64 * wave + lane) * 4u, rsS, 0);
    };
    bool has_next = false;
    // instruction i (0..kHalf-1) of half `half` of a stage of kind KIND; the
    // T stage's first half also carries the s table
    auto dma_grp = [&](auto kind_c, int u, int soff, int half, int i) {
        constexpr int KIND = decltype(kind_c)::value;
        if constexpr (KIND == kMain) {
            dma_k(u, uint32_t(soff), half * kHalf + i);
        } else if constexpr (KIND == kT) {
            if (i < kLoraHalf && R > 0) dma_lora(true, soff, half * kLoraHalf + i);
            if (half == 0 && i == kLoraHalf) dma_scale();
        } else if constexpr (KIND == kLA) {
            if (i < kLaHalf && R > 0) dma_lora(false, soff, half * kLaHalf + i);
        } else {
            if (has_next) dma_k(0, uint32_t(soff), half * kHalf + i);
        }
    };
    // s_waitcnt for "stage t + 1 has landed" when stage t + 2 is of kind NEXT2
    auto wait_next = [&](auto next2_c) {
        constexpr int NEXT2 = decltype(next2_c)::value;
        if constexpr (NEXT2 == kMain) {
            wait_vmcnt_lgkm0<C::DMA_PER_STAGE>();
        } else if constexpr (NEXT2 == kT) {
            if (R > 0) {
                wait_vmcnt_lgkm0<2 * kLoraHalf + 1>();
            } else {
                wait_vmcnt_lgkm0<1>();
            }
        } else {
            if (R > 0) {
                wait_vmcnt_lgkm0<2 * kLaHalf>();
            } else {
                wait_vmcnt_lgkm0<0>();
            }
        }
    };
    using IMain = std::integral_constant<int, kMain>;
    using IT = std::integral_constant<int, kT>;
    using ILA = std::integral_constant<int, kLA>;
    using INext0 = std::integral_constant<int, kNext0>;

    // byte offsets of slots t % 3, (t + 1) % 3, (t + 2) % 3, rotated per stage
    int cur = 0, nxt = C::STAGE, aft = 2 * C::STAGE;
    // one stage: G2 = kind of stage t + 2 (second half issued here), G3 = kind
    // of stage t + 3 (first half issued here)
    auto stage = [&](int t, auto g2, auto g3) {
#pragma unroll
        for (int k = 0; k < kS; ++k) {
            mma(fr[0], k);
            if (k < kR2) {
                read_n(cur, 1, fr[1], 2 * k);
                read_n(cur, 1, fr[1], 2 * k + 1);
            }
            if (k >= kR2) {
                // stage t + 2's kPartB + kHalf DMAs over the slots after the reads
                constexpr int kSlots = kS - kR2;
#pragma unroll
                for (int d = k - kR2; d < kPartB + kHalf; d += kSlots) {
                    if (d < kPartB) {
                        dma_grp(g2, t + 2, aft, 0, kPartA + d);
                    } else {
                        dma_grp(g2, t + 2, aft, 1, d - kPartB);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int k = 0; k < kBar; ++k) {
            mma(fr[1], k);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_next(g2);  // stage t + 1 has landed
        block_barrier();
#pragma unroll
        for (int k = kBar; k < kS; ++k) {
            mma(fr[1], k);
            if (k - kBar < kR2) {
                read_n(nxt, 0, fr[0], 2 * (k - kBar));
                read_n(nxt, 0, fr[0], 2 * (k - kBar) + 1);
            }
            if (k - kBar - kR2 >= 0 && k - kBar - kR2 < kPartA)
                dma_grp(g3, t + 3, cur, 0, k - kBar - kR2);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int freed = cur;
        cur = nxt;
        nxt = aft;
        aft = freed;
    };

    const bool vec_ok = (N & 7) == 0;
    // Y as a buffer: 32-bit offsets (M N < 2^31) keep the store addressing cheap
    const __amdgpu_buffer_rsrc_t rsY =
        __builtin_amdgcn_make_buffer_rsrc(Y, 0, int(uint32_t(M) * uint32_t(N) * 2u), kRsrcWord3);
    const float* s_lds = reinterpret_cast<const float*>(smem + C::SCALE_OFF);
    char* ep = smem + kEpiOff + wave * kEpiWave;

    int v = blockIdx.x;
    {
        int tm, tn;
        tile_of(v, tiles_m, tiles_n, tm, tn);
        m0 = tm * BM;
        n0 = tn * TN;
    }
    set_tile_offsets(m0, n0);
    __builtin_amdgcn_s_waitcnt(0);
    for (int k = 0; k < C::DMA_PER_STAGE; ++k) dma_k(0, uint32_t(cur), k);  // first tile's stage 0

    for (; v < ntiles; v += gridDim.x) {
        // stage 0 of this tile is in flight into slot `cur`
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[a][b] = f32x16{};
        for (int k = 0; k < C::DMA_PER_STAGE; ++k) dma_k(1, uint32_t(nxt), k);
        if (nk > 2) {
            for (int i = 0; i < kPartA; ++i) dma_grp(IMain{}, 2, aft, 0, i);
            wait_vmcnt<C::DMA_PER_STAGE + kPartA>();  // stage 0 has landed
        } else {
            for (int i = 0; i < kPartA; ++i) dma_grp(IT{}, 2, aft, 0, i);
            // the T stage's first kPartA instructions: T rows, and s unless it
            // is in part B
            constexpr int kScaleA = kPartA > kLoraHalf ? 1 : 0;
            constexpr int kTA = kPartA < kLoraHalf ? kPartA : kLoraHalf;
            if (R > 0) {
                wait_vmcnt<C::DMA_PER_STAGE + kTA + kScaleA>();
            } else {
                wait_vmcnt<C::DMA_PER_STAGE + kScaleA>();
            }
        }
        block_barrier();
#pragma unroll
        for (int n = 0; n < kReads; ++n) read_n(cur, 0, fr[0], n);

        for (int t = 0; t < nk - 3; ++t) stage(t, IMain{}, IMain{});
        if (nk >= 3) stage(nk - 3, IMain{}, IT{});
        stage(nk - 2, IT{}, ILA{});
        // the current tile's stage loads are all issued: point the offsets at
        // the next tile, whose stage 0 goes out from here on
        const int vn = v + gridDim.x;
        has_next = vn < ntiles;
        int m0n = m0, n0n = n0;
        if (has_next) {
            int tm, tn;
            tile_of(vn, tiles_m, tiles_n, tm, tn);
            m0n = tm * BM;
            n0n = tn * TN;
            set_tile_offsets(m0n, n0n);
        }
        stage(nk - 1, ILA{}, INext0{});
        // rotation after the last stage: cur = T, nxt = LA, aft = next stage 0
        for (int i = kPartA; i < kHalf; ++i) dma_grp(INext0{}, 0, aft, 0, i);
        for (int i = 0; i < kHalf; ++i) dma_grp(INext0{}, 0, aft, 1, i);
        if (has_next) {
            wait_vmcnt_lgkm0<C::DMA_PER_STAGE>();  // LA landed (next stage 0 may fly)
        } else {
            wait_vmcnt_lgkm0<0>();
        }
        __syncthreads();  // LoRA operands landed; all waves done with the stage slots

        // ---- y = s * acc + T LA^T: rows scaled by s, then the LoRA up-projection
        // accumulated on top, with T as stored (no bf16 rounding of T / s)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 sv = *reinterpret_cast<const f32x4*>(s_lds + wm * 128 + 32 * a + 8 * j + 4 * h);
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[a][b][4 * j + i] *= sv[i];
            }
        if (R > 0) {
            const char* Ts = smem + cur;
            const char* Ls = smem + nxt;
            // T is dense; it is fed to the same SMFMAC as two exactly-2:4
            // halves with fixed positions (0,1 -> code 0x4; 2,3 -> code 0xE per
            // group): over channels [16h, 16h+16) of a 32-rank step the even
            // dwords of the row are positions 0,1 of each group and the odd
            // dwords positions 2,3.  LA supplies the B operand exactly as W
            // does in the main loop.
            const int nks = (R + 31) / 32;  // 1 or 2 (R <= 64)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks >= nks) break;
                const int cb0 = 16 * ((4 * ks + h) ^ s128), cb1 = 16 * ((4 * ks + 2 + h) ^ s128);
                const int ca0 = 16 * ((4 * ks + 2 * h) ^ s128);
                const int ca1 = 16 * ((4 * ks + 2 * h + 1) ^ s128);
                bf16x16 bl[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int row = (wn * WC + 32 * b + r) * 128;
                    const bf16x8 lo = lds_read<bf16x8>(Ls, row + cb0);
                    const bf16x8 hi = lds_read<bf16x8>(Ls, row + cb1);
                    bl[b] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11,
                                                    12, 13, 14, 15);
                }
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int row = (wm * 128 + 32 * a + r) * 128;
                    const u32x4 t0 = lds_read<u32x4>(Ts, row + ca0);
                    const u32x4 t1 = lds_read<u32x4>(Ts, row + ca1);
                    const bf16x8 te = __builtin_bit_cast(bf16x8, u32x4{t0.x, t0.z, t1.x, t1.z});
                    const bf16x8 to = __builtin_bit_cast(bf16x8, u32x4{t0.y, t0.w, t1.y, t1.w});
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        acc[a][b] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                            te, bl[b], acc[a][b], 0x4444, 0, 0);
                        acc[a][b] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                            to, bl[b], acc[a][b], 0xEEEE, 0, 0);
                    }
                }
            }
        }

        // ---- epilogue: interior tiles straight from the accumulators, edge
        // tiles (columns past N, or N % 8 != 0) through the LDS staging rows
        if (vec_ok && n0 + TN <= N) {
            store_block_direct<NB>(acc, rsY, N, m0 + wm * 128, n0 + wn * WC);
        } else {
            // ---- epilogue: y = acc, bf16, 8 rows at a time through LDS ----------
            // Rows of a 32 x 32 tile held by this lane: 8 (e / 4) + 4 h + e % 4, so
            // round (a, j) takes e = 4j .. 4j+3 (rows 8j .. 8j+7 of row block a).
            // Staging rows 4..7 have their 128-byte halves swapped so the two
            // halves of the wave write different banks.
    #pragma unroll
            for (int a = 0; a < 4; ++a) {
    #pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rbase = wm * 128 + 32 * a + 8 * j;  // tile row of staging row 0
    #pragma unroll
                    for (int b = 0; b < NB; ++b)
    #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int lr = 4 * h + i;  // staging row 0..7
                            *reinterpret_cast<uint16_t*>(ep + lr * 256 + (((32 * b + r) * 2) ^ (h << 7))) =
                                __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[a][b][4 * j + i]));
                        }
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    // lane -> staging row lane / 8, 16 columns from (lane % 8) * 16
                    // (of the wave's WC columns)
                    const int el = fresh_lane();
                    const int srow = el >> 3;
                    const int orow = m0 + rbase + srow;
                    const int ocol = n0 + wn * WC + (el & 7) * 16;
                    if (orow < M && (el & 7) < 2 * NB) {
                        const int sb = srow * 256 + (((el & 7) * 32) ^ ((srow >> 2) << 7));
    #pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const u32x4 w4 = lds_read<u32x4>(ep, sb + 16 * i);
                            const int col = ocol + 8 * i;
                            const uint32_t yoff = (uint32_t(orow) * uint32_t(N) + uint32_t(col)) * 2u;
                            if (vec_ok && col + 8 <= N) {
                                __builtin_amdgcn_raw_buffer_store_b128(w4, rsY, yoff, 0, 0);
                            } else {
                                const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
    #pragma unroll
                                for (int q2 = 0; q2 < 8; ++q2)
                                    if (col + q2 < N)
                                        __builtin_amdgcn_raw_buffer_store_b16(
                                            uint16_t(w[q2 >> 1] >> (16 * (q2 & 1))), rsY,
                                            yoff + 2u * q2, 0, 0);
                            }
                        }
                    }
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
            }
        }
        __syncthreads();  // T / LA slots, s and the staging rows are free
        // the next tile: its stage 0 is in slot `aft`
        const int t_slot = cur;
        cur = aft;
        aft = nxt;
        nxt = t_slot;
        m0 = m0n;
        n0 = n0n;
    }
}

}  // namespace

lynx_status launch_gemm_sparse_tiled(const uint16_t* values, const uint8_t* meta,
                                     const float* scale, const uint16_t* T, const uint16_t* W,
                                     const uint16_t* LA, uint16_t* Y, int M, int N, int K, int R,
                                     hipStream_t stream) {
    // persistent: one workgroup per compute unit (the kernel's LDS allows one).
    // Tile width 256 or 192: the one whose rounds of tiles over the compute
    // units cost less (rounds x width; ties to 256), which removes most of the
    // idle last round when the 256-wide tiles do not divide evenly.
    int cus = 0;
    if (device_cu_count(&cus) != LYNX_OK) return LYNX_ERR_DEVICE;
    const long tm = (M + BM - 1) / BM;
    auto tiles_for = [&](int tn) { return tm * ((N + tn - 1) / tn); };
    auto cost = [&](int tn) { return (tiles_for(tn) + cus - 1) / cus * tn; };
    const bool narrow = cost(192) < cost(256);
    const long tiles = tiles_for(narrow ? 192 : 256);
    const int grid = int(tiles < cus ? tiles : cus);
    if (narrow) {
        hipLaunchKernelGGL(gemm_sparse32<3>, dim3(grid), dim3(NT), 0, stream, values, meta, scale,
                           T, W, LA, Y, M, N, K, R);
    } else {
        hipLaunchKernelGGL(gemm_sparse32<4>, dim3(grid), dim3(NT), 0, stream, values, meta, scale,
                           T, W, LA, Y, M, N, K, R);
    }
    return launch_status();
}

}  // namespace lynx
