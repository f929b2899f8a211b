// internal.h -- declarations shared by the host half (vqmlp_host.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vqmlp {

// ---- packed VQ3 layout (version 1); see include/vqmlp.h for the byte-level description
constexpr uint32_t kMagic = 0x50335156u;  // "VQ3P" little-endian
constexpr int kHeaderBytes = 256;
constexpr int kTilePairs = 16;            // row pairs per tile (one matrix-core operand height)
constexpr int kTileRows = 2 * kTilePairs; // 32 output rows
constexpr int kTileCols = 64;             // input columns per tile (4 steps of 16)
constexpr int kTileBytes = 768;           // 64 lanes x 12 bytes (16 six-bit codes)
constexpr int kGroupRows = 8;             // rows sharing one codebook
constexpr int kCodebook = 64;             // entries per codebook (2 x binary16 each)

struct PackedHeader {
    uint32_t magic, version, N, K, group_rows, entries, kind, reserved;
    uint64_t codes_off, codes_bytes, cb_off, cb_bytes, sc_off, sc_bytes, total;
};
static_assert(sizeof(PackedHeader) <= kHeaderBytes, "header");

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Host only: record the text of a failure for vqmlp_last_error() (this thread) and return st.
int set_last_error(int st, const char* fmt, ...);
// Host only: the allocation-free forward's per-device scratch array (noalloc.hip): fetch this
// device's address and zero it, once per device (called by vqmlp_create).
void noalloc_setup();

struct VQ3View {          // device pointers into one packed buffer
    const uint8_t* codes;     // tiles
    const uint32_t* cb;       // [N/8][64] dwords: (binary16 even row) | (binary16 odd row) << 16
    const uint16_t* sc;       // [N]
    int N, K;
};

// ---- skinny path (T <= 8)
constexpr int kSkinnyT = 8;            // rows of the matrix-core operand (8 tokens x 2 components)
constexpr int kSkinnyWaves = 16;       // waves per workgroup, each owning a K range
constexpr int kSkinnyMaxTPW = 5;       // 64-column tiles per wave held in registers

// ---- launchers (kernels.hip).  All return hipError_t of the launch.
hipError_t launch_dequant(const VQ3View& m, float* w, hipStream_t s);

// out[t][.] = R(x . s . sign) for a binary16 or float input, Hadamard blocks of b (a power of
// two up to 1024; 1 = no rotation).  mode: 0 = FP32 row-major [T][n], 1 = binary16 row-major
// [T][n].
hipError_t launch_rotate(int T, int n, int b, const void* x, int x_is_f32, const uint16_t* s,
                         const int8_t* sign, void* out, int mode, hipStream_t st);
// Reads bytes (a multiple of 16) of buf once, 16-byte loads, contiguous share per workgroup.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int cus,
                              hipStream_t st);

// ---- scalar-LUT projection for T <= 8 (K <= kLut8MaxK): y = sc . (W_lut x~) + U z
constexpr int kLut8MaxK = 5120;
struct Lut8Args {
    const uint32_t* codes;  // [N][K * bits / 32] row-major code words
    const uint16_t* lut;    // [N / 8][2^bits] binary16
    const uint16_t* sc;     // [N] binary16 row scales
    const uint16_t* x;      // x~ [T][K] binary16
    uint16_t* y;            // [T][N] binary16
    const uint16_t* U;      // [N][r] binary16 (r > 0)
    const float* zp;        // [nch][8][r] fp32 partial sums of z = V x~ (r > 0), summed in order
    int bits, N, K, T, r, nch;
};
hipError_t launch_lut8(const Lut8Args& a, hipStream_t st);
// 2x16 vector-LUT projection at T <= 8: y[t][r] = sc[r] * sum_j cb[r/8][code[r/2][j]][r%2] x[t][j]
// (x as given; FP32 accumulation, one rounding).  N % 32 == 0, K % 32 == 0, K <= kVq2MaxK.
// K split: grid.y = nsplit slices of K columns each (the matrix and x have ldk = nsplit * K
// columns); a split product writes unscaled FP32 partial sums instead of y.
constexpr int kVq2MaxK = 5120;
struct Vq2Args {
    const uint32_t* codes;  // [N/2][ldk/8] words, code j of a pair row at bits 4 (j % 8) of word j / 8
    const uint32_t* cb;     // [N/8][16] centroids, binary16 (component 0) | (component 1) << 16
    const uint16_t* sc;     // [N] binary16 row scales
    const uint16_t* x;      // [T][ldk] binary16
    uint16_t* y;            // [T][N] binary16 (out32 == nullptr)
    float* out32;           // unscaled sums: out32[split * o32_s + t * o32_t + row] (or nullptr)
    int N, K, T;            // K: columns of one slice
    int ldk, nsplit;        // full K = nsplit * K
    int o32_t, o32_s;
    // A second matrix over the same x (gate and up in one launch; out32 required): grid rows
    // nsplit .. 2 nsplit - 1 take it and write their planes at out32 + o32_m.  NULL: one matrix.
    const uint32_t* codes2;
    const uint32_t* cb2;
    const uint16_t* sc2;
    int o32_m;
};
hipError_t launch_vq2_8(const Vq2Args& a, hipStream_t st);
// Pre-pass of the T <= 8 projection: x~ = R_K(x . s . sign) ([T][K] binary16, Hadamard block hb,
// 1 = none) and, for r > 0, the partial sums zp[c][t][j] = sum over part c of V[j][k] x~[t][k]
// (rotated in chunks of lut8_chunk(K, hb) columns, summed in parts of at most 256 of them:
// lut8_planes(K, hb) planes; x~ rounded to binary16 first).
int lut8_chunk(int K, int hb);
// Greedy argmax of a scalar-LUT output head (r == 0): out_idx[t] = the lowest row of the largest
// logit sc . (W_lut x~) of token t (x~ = a.x as given), out_val[t] that logit (FP32, may be NULL).
// pval / pidx: lut8_argmax_grid(N, cus) x 8 partial bests.
constexpr int kArgmaxMaxGroups = 1024;  // workgroups of the argmax head at most
int lut8_argmax_grid(int N, int cus);
hipError_t launch_lut8_argmax(const Lut8Args& a, int cus, float* pval, int* pidx, int* out_idx,
                              float* out_val, hipStream_t st);
int lut8_planes(int K, int hb);
hipError_t launch_lut8_pre(int T, int K, int hb, const uint16_t* x, const uint16_t* s,
                           const int8_t* sign, const uint16_t* V, int r, uint16_t* xt, float* zp,
                           hipStream_t st);

// ---- fused persistent forward (T <= 8): the whole MLP in one launch
// Control block (kCtlHdr 32-bit words, zero before the first call): word 0 is the item queue
// head and word 1 counts finished workgroups (both back to zero after each call), word 2
// collects error bits, word 3 is the call epoch.  Every hand-off between workgroups is a 64-bit word carrying the
// call's tag (epoch + 1) beside 32 bits of data, so readers need no separate ready flags.
enum { kCtlQueue = 0, kCtlExit = 1, kCtlError = 2, kCtlEpoch = 3, kCtlHdr = 16 };
struct FusedArgs {
    VQ3View gate, up, down;
    int H, I, T;
    int bh, bi;          // Hadamard blocks
    int rc;              // columns per input-rotation item (multiple of bh)
    int fu;              // intermediate rows per rotation unit (max(bi, 32))
    int n_r, n_g, nsl, nqd, n_fu, total;  // item counts: rotation, gate/up, down slices x pairs
    float norm_h, norm_i;
    const uint16_t* x;       // [T][H] binary16
    const uint16_t* s;       // [H] input scale
    const int8_t* sign_h;    // [H] or NULL
    const int8_t* sign_i;    // [I] or NULL
    uint16_t* y;             // [T][H] binary16
    uint32_t* ctl;           // control block (kCtlHdr words)
    uint64_t* xb;            // [2][8][H/2] rotated input, binary16 pairs, tagged; rows past T
                             // zero; two buffers used by call parity
    uint64_t* act;           // [8][I] silu(g) u sign, FP32 bits, tagged
    uint64_t* ab;            // [2][8][I/2] rotated intermediate, binary16 pairs, tagged
    uint64_t* part;          // [nsl][8][H] tagged FP32 partial sums of the down projection
    unsigned spin_limit;     // bound of every wait (then the error word records it)
    int dyn;                 // items after the first two rounds from the queue (else round-robin)
};
inline size_t fused_ctl_words() { return size_t(kCtlHdr); }
int fused_tpw(int H);  // tiles per wave of the fused kernel for hidden size H (0 = unsupported)
hipError_t launch_fused(const FusedArgs& a, int tpw, int grid, hipStream_t st);

// ---- tiled matrix-core path (T > 8): decoders, epilogues, kinds
enum { kDecVQ3 = 0, kDecLUT2 = 1, kDecLUT4 = 2, kDecDense = 3, kDecVQ2 = 4 };
enum { kEgGateUp32 = 0, kEgGateUpRot = 1, kEgScale16 = 2, kEgLUT = 3, kEgPlain32 = 4, kEgPart2 = 5,
       kEgLUTPlane = 6 };
enum {
    kGemmVQ3GateUp = 0,     // gate+up -> a fp32 [T][N] (sign applied)
    kGemmVQ3GateUpRot = 1,  // gate+up -> rotated a binary16 [T][N] (128-wide blocks)
    kGemmVQ3Down = 2,       // down -> y binary16 [T][N]
    kGemmLUT2 = 3,          // scalar LUT 2-bit + rank-r factors -> y binary16
    kGemmLUT4 = 4,          // scalar LUT 4-bit + rank-r factors -> y binary16
    kGemmDense32 = 5,       // dense binary16 rows -> fp32 [T][N]
    kGemmVQ3DownSplit = 6,  // down, K split -> unscaled fp32 partials [ksplit][T][N]
    kGemmVQ3GateUpSplit = 7 // gate+up, K split -> unscaled fp32 g, u planes [ksplit][T][2][N]
};
struct GemmArgs {
    int kind, N, K, T;
    int ksplit;                // K splits (blockIdx.z): down-split and dense kinds; 0/1 = none
    const uint16_t* x;         // [T][K] binary16
    const uint8_t* codes[2];   // packed code sections
    const uint32_t* cb[2];     // VQ3 codebooks / LUT tables (binary16 pairs)
    const uint16_t* sc[2];     // row scales
    const uint16_t* dense;     // dense rows [N][K]
    const int8_t* sign;        // intermediate rotation sign (gate+up)
    float* out32;
    uint16_t* out16;
    const float* z;            // rank-r activations [T][r]
    const uint16_t* U;         // rank-r factor [N][r]
    int r;
    float norm;                // 1/sqrt(rotation block); K-split planes of vq3mm: plane scale
    int ldo;                   // output row stride (0 = N)
    int vq2;                   // the VQ3 kinds on 2x16 matrices (codes [N/2][K/8] words,
                               // 16 centroids per 8 rows): tiled kernels with the 2x16 decoder
    int bm64;                  // K-split gate/up of vq3mm above 64 rows: 64-token tiles
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
// VQ3 products for T > 32 rows with the weights decoded in registers (vq3mm.hip): gate/up kinds
// (two matrices), down and scalar-LUT kinds (one).  Tile of one workgroup of a product of this
// kind with T rows: bm tokens x bn rows.
struct Vq3Tile {
    int bm, bn;
};
Vq3Tile vq3mm_tile(int kind, int T);
hipError_t launch_vq3mm(const GemmArgs& a, hipStream_t st);
constexpr int kVq3mmMinT = 33;  // launch_gemm sends VQ3 kinds with at least this many rows there
// K splits for a product of this kind and shape on `cus` CUs (1 = none).  A split product
// writes unscaled FP32 planes [ksplit][T][N]; the reductions below finish it.
int gemm_split(int kind, int N, int K, int T, int cus);
hipError_t launch_split_reduce(int T, int N, int splits, const float* part, const uint16_t* sc,
                               uint16_t* y, hipStream_t st);  // y = sc . sum (sc null: 1)
hipError_t launch_split_sum(int n, int splits, const float* part, float* out, hipStream_t st);
// a = silu(sc_g sum g) (sc_u sum u) sign from K-split gate/up planes [splits][T][2][N]; rotate:
// 128-wide rotation to binary16 out16 [T][ldo], else FP32 out32 [T][ldo]
hipError_t launch_gateup_combine(int T, int N, int splits, const float* part,
                                 const uint16_t* scg, const uint16_t* scu, const int8_t* sign,
                                 int rotate, float norm, int ldo, uint16_t* out16, float* out32,
                                 hipStream_t st);

}  // namespace vqmlp
