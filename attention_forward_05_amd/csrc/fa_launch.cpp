// fa_launch.cpp -- loads the gfx950 attention kernels (assembled from the
// generators in attention_forward_05_amd/asm and embedded in this library as
// a code object) and launches them.
//
// Two kernel shapes, for D = 64 and 128: four waves on 256-row query tiles,
// and, when the 512-row tiles alone give every compute unit an item (and
// each item with keys spans at least 3 key tiles), eight waves (two per
// SIMD, alternating MFMA and softmax phases) on 512-row tiles, which halves
// the K/V traffic into LDS per FLOP and streams K/V tiles across items.
// For D = 128, when the 512-row items would leave compute units idle, the
// key ranges are long and the caller passed a workspace, each item's keys
// are split into 2..16 ranges whose partial results (in that workspace) a
// combine kernel (fa_combine.hip) merges.  The library itself allocates no
// device memory.
//
// The kernels are persistent: the grid has G = min(items, compute units)
// workgroups, one per CU, and workgroup g takes item r*G + (g or G-1-g,
// alternating by round r) of the (batch, q-head, query tile) items, which the
// kernel orders longest first.  Workgroups are handed to the 8
// XCDs round-robin by id, so within a round each XCD sees one residue of the
// head slot mod 8; the kernel maps slot s to head (s % 8) * (Hq / 8) + s / 8
// when Hq % 8 == 0, so each XCD serves a contiguous run of heads (whole GQA
// groups) whose K/V its L2 keeps.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_kernel.h"

extern "C" const unsigned char fa_hsaco_data[];
extern "C" const unsigned long fa_hsaco_size;

namespace fa {
namespace {

constexpr int kBM = 256;       // query rows per workgroup (four-wave kernels)
constexpr int kBM8 = 512;      // query rows per workgroup (eight-wave kernels)
constexpr int kBN = 64;        // keys per tile
constexpr int kMaxDevices = 64;

struct alignas(8) KernArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t B, Sq, Skv, Hq, Hkv, causal;
  float c;
  uint32_t nq_grid;  // query tiles | workgroups << 16
  uint32_t gmagic;  // hk = (hq * gmagic) >> 20
  uint32_t hq_xcd;  // Hq / 8 when Hq % 8 == 0, else 0
  uint32_t log2split;  // split kernels: log2 of the key ranges per item
  uint32_t pad[3];
};
static_assert(sizeof(KernArgs) == 96, "kernarg layout of the generated kernels");

constexpr int kKernels = 18;
const char* kNames[kKernels] = {"fa_fwd_bf16_d128_gfx950",     "fa_fwd_bf16_d64_gfx950",
                                "fa_fwd_f16_d128_gfx950",      "fa_fwd_f16_d64_gfx950",
                                "fa_fwd_bf16_d128_x8_gfx950",  "fa_fwd_f16_d128_x8_gfx950",
                                "fa_fwd_bf16_d128_x8s_gfx950", "fa_fwd_f16_d128_x8s_gfx950",
                                "fa_fwd_bf16_d64_x8_gfx950",   "fa_fwd_f16_d64_x8_gfx950",
                                // backward: dK/dV then dQ, each (bf16, f16) x (D 128, 64)
                                "fa_bwd_dkv_bf16_d128_gfx950", "fa_bwd_dkv_bf16_d64_gfx950",
                                "fa_bwd_dkv_f16_d128_gfx950",  "fa_bwd_dkv_f16_d64_gfx950",
                                "fa_bwd_dq_bf16_d128_gfx950",  "fa_bwd_dq_bf16_d64_gfx950",
                                "fa_bwd_dq_f16_d128_gfx950",   "fa_bwd_dq_f16_d64_gfx950"};
constexpr int kBwdFirst = 10;

// Arguments of the generated backward kernels (fa_bwd_gen.py).
struct alignas(8) BwdKernArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* l2;     // LSE * log2(e) per query row
  const float* delta;  // rowsum(O * dO) per query row
  void* dq;
  void* dk;
  void* dv;
  int32_t B, Sq, Skv, Hq, Hkv, causal;
  float c;       // scale * log2(e)
  float scale;
  uint32_t nqb;     // dQ: 128-row query blocks
  uint32_t gmagic;  // hk = (hq * gmagic) >> 20
  uint32_t group;   // Hq / Hkv
  uint32_t pad[3];
};
static_assert(sizeof(BwdKernArgs) == 128, "kernarg layout of the generated backward kernels");

struct DeviceKernels {
  bool loaded = false;
  hipModule_t mod = nullptr;
  hipFunction_t fn[kKernels] = {};
  int cus = 0;  // compute units of the device
};

std::mutex g_mu;
DeviceKernels g_dev[kMaxDevices];

hipError_t kernels_for_current_device(DeviceKernels** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceKernels& d = g_dev[dev];
  if (!d.loaded) {
    e = hipModuleLoadData(&d.mod, fa_hsaco_data);
    if (e != hipSuccess) return e;
    for (int i = 0; i < kKernels; ++i) {
      e = hipModuleGetFunction(&d.fn[i], d.mod, kNames[i]);
      if (e != hipSuccess) return e;
    }
    e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (d.cus < 1) d.cus = 1;
    d.loaded = true;
  }
  *out = &d;
  return hipSuccess;
}

}  // namespace

int launch_bwd(const BwdLaunchArgs& a) {
  DeviceKernels* dk = nullptr;
  if (kernels_for_current_device(&dk) != hipSuccess) return FA_ERR_HIP;
  uint32_t magic = 0;
  if (!group_magic(a.Hq, a.Hkv, &magic)) return FA_ERR_UNSUPPORTED;
  if (launch_bwd_delta(a) != hipSuccess) return FA_ERR_HIP;
  const size_t rows = (size_t)a.B * a.Hq * a.Sq;
  BwdKernArgs k;
  memset(&k, 0, sizeof(k));
  k.q = a.q;
  k.k = a.k;
  k.v = a.v;
  k.dout = a.dout;
  k.l2 = a.ws;
  k.delta = a.ws + rows;
  k.dq = a.dq;
  k.dk = a.dk;
  k.dv = a.dv;
  k.B = a.B;
  k.Sq = a.Sq;
  k.Skv = a.Skv;
  k.Hq = a.Hq;
  k.Hkv = a.Hkv;
  k.causal = a.causal;
  k.c = a.c;
  k.scale = a.scale;
  k.nqb = (uint32_t)((a.Sq + 127) / 128);
  k.gmagic = magic;
  k.group = (uint32_t)(a.Hq / a.Hkv);
  const int var = (a.dtype == DType::kBF16 ? 0 : 2) + (a.D == 128 ? 0 : 1);
  size_t size = sizeof(k);
  void* cfg[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, &k, HIP_LAUNCH_PARAM_BUFFER_SIZE, &size,
                 HIP_LAUNCH_PARAM_END};
  // dK/dV: a workgroup per (kv-head, batch, 128-key block); dQ: per (q-head,
  // batch, 128-row query block from the last).  The block index varies
  // slowest, so the workgroups with the most work start first (a causal
  // call's first keys and last rows see the most of the other side).
  hipError_t e = hipModuleLaunchKernel(dk->fn[kBwdFirst + var], (unsigned)a.Hkv, (unsigned)a.B,
                                       (unsigned)((a.Skv + 127) / 128), 256, 1, 1, 0, a.stream,
                                       nullptr, cfg);
  if (e != hipSuccess) return FA_ERR_HIP;
  e = hipModuleLaunchKernel(dk->fn[kBwdFirst + 4 + var], (unsigned)a.Hq, (unsigned)a.B, k.nqb,
                            256, 1, 1, 0, a.stream, nullptr, cfg);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

bool group_magic(int Hq, int Hkv, uint32_t* magic) {
  const uint32_t g = (uint32_t)(Hq / Hkv);
  const uint64_t m = (1ull << 20) / g + 1;
  for (int hq = 0; hq < Hq; ++hq) {
    const uint64_t p = (uint64_t)hq * m;
    if (p >> 32) return false;
    if ((uint32_t)(p >> 20) != (uint32_t)hq / g) return false;
  }
  *magic = (uint32_t)m;
  return true;
}

hipError_t launch_kernel(DeviceKernels* dk, const LaunchArgs& a, int variant, bool x8, int l2s);

int64_t work_items(int B, int Sq, int Hq) {
  return (((int64_t)Sq + kBM - 1) / kBM) * B * Hq;
}

int query_tiles(int Sq) { return (int)(((int64_t)Sq + kBM - 1) / kBM); }

int64_t min_item_tiles(int Sq, int Skv, int causal) {
  // Key ranges grow with the query tile, so the first 512-row query tile
  // with a visible key is the shortest.
  if (!causal) return key_tiles(Skv);
  const int64_t off = (int64_t)Skv - Sq;
  for (int64_t q0 = 0; q0 < Sq; q0 += kBM8) {
    const int64_t end = std::min<int64_t>(Skv, std::min<int64_t>(q0 + kBM8, Sq) + off);
    if (end > 0) return (end + kBN - 1) / kBN;
  }
  return 0;
}

bool use_eight_waves(int B, int Sq, int Skv, int Hq, int D, int causal, int cus) {
  if ((D != 128 && D != 64) || (((int64_t)Sq + kBM8 - 1) / kBM8) * B * Hq < cus) return false;
  // The eight-wave kernel streams K/V tiles across consecutive items and
  // needs every item with a visible key to span at least 3 key tiles.
  const int64_t n = min_item_tiles(Sq, Skv, causal);
  return n == 0 || n >= 3;
}

int split_log2(int B, int Sq, int Skv, int Hq, int D, int causal, int cus) {
  if (D != 128) return 0;
  const int64_t items = (((int64_t)Sq + kBM8 - 1) / kBM8) * B * Hq;
  if (items >= cus) return 0;
  const int64_t n = min_item_tiles(Sq, Skv, causal);
  if (n == 0) return 0;
  // The fewest key ranges (a power of two, at most 16) that give every
  // compute unit an item, while each range keeps at least 16 key tiles:
  // below that the partial results' traffic outweighs the gain.  When the
  // four-wave kernel's 256-row items already cover the compute units, split
  // only ranges of at least 64 key tiles: on shorter ones writing and
  // merging the partial results costs more than the eight-wave kernel's
  // faster loop saves.
  const int64_t min_range = work_items(B, Sq, Hq) >= cus ? 64 : 16;
  int l = 0;
  while (l < 4 && (items << l) < cus) ++l;
  while (l > 0 && n < (min_range << l)) --l;
  return l;
}
int key_tiles(int Skv) { return (int)(((int64_t)Skv + kBN - 1) / kBN); }

size_t split_ws_bytes(int B, int Sq, int Hq, int D, int ranges) {
  if (ranges <= 1) return 0;
  const size_t rows = (size_t)B * Hq * Sq * (size_t)ranges;
  return rows * 4 * (size_t)(D + 1);
}

namespace {

// Tile kernels: rows per item and keys per tile.
int tile_rows(bool keys) { return keys ? 32 : 128; }
int tile_keys(bool keys, int D) { return keys ? 128 : (D == 256 ? 32 : 64); }

// Key tiles of the tile kernel's shortest item with a visible key (0: none).
int64_t tile_min_tiles(int Sq, int Skv, int causal, int gp, int rows, int tk) {
  if (!causal) return (Skv + tk - 1) / tk;
  const int64_t off = (int64_t)Skv - Sq;
  const int64_t nrows = (int64_t)Sq * gp;
  for (int64_t n0 = 0; n0 < nrows; n0 += rows) {
    const int64_t last_i = (std::min<int64_t>(n0 + rows, nrows) - 1) / gp;
    const int64_t end = std::min<int64_t>(Skv, last_i + 1 + off);
    if (end > 0) return (end + tk - 1) / tk;
  }
  return 0;
}

}  // namespace

Plan make_plan(int B, int Sq, int Skv, int Hq, int Hkv, int D, int causal, int cus,
               bool allow_split) {
  Plan p;
  p.packed = false;
  const int g = Hq / Hkv;
  // Decode-shaped calls (a few query rows): the q-heads of a kv-head share
  // one block of rows, so K and V are read once per kv-head; with at most 32
  // such rows the four waves split the keys instead of the rows.  Head
  // dimension 256 has only the tile kernel.
  const bool decode = D != 256 && Sq <= 64;
  // Causal D = 64 calls that the eight-wave kernel does not take and whose
  // 256-row query tiles fill at most one round: one round of causal items
  // is only as fast as its longest; the tile kernel's 128-row items run in
  // two rounds, longest first, which balances them (3-7% faster measured).
  const bool causal64 = D == 64 && causal && !decode && work_items(B, Sq, Hq) <= cus &&
                        !use_eight_waves(B, Sq, Skv, Hq, D, causal, cus);
  if (D == 256 || decode || causal64) {
    p.packed = decode;
    const int gp = decode ? g : 1;
    const bool keys = decode && (int64_t)Sq * g <= 32;
    p.kernel = keys ? kTileKeys : kTileRows;
    const int rows = tile_rows(keys), tk = tile_keys(keys, D);
    const int64_t heads = decode ? Hkv : Hq;
    const int64_t items = (int64_t)B * heads * (((int64_t)Sq * gp + rows - 1) / rows);
    const int64_t n = tile_min_tiles(Sq, Skv, causal, gp, rows, tk);
    // Split key ranges (with a workspace) until the items cover the compute
    // units (twice over for the memory-bound key split), keeping at least 4
    // (keys) or 8 (rows) key tiles per range; at most 64 ranges.
    const int64_t target = keys ? 2 * (int64_t)cus : cus;
    const int64_t min_tiles = keys ? 4 : 8;
    int ns = 1;
    if (allow_split)
      while (ns < 64 && items * ns < target && n >= min_tiles * 2 * ns) ns *= 2;
    p.ranges = ns;
    p.ws_bytes = split_ws_bytes(B, Sq, Hq, D, ns);
    return p;
  }
  const int l2s = allow_split ? split_log2(B, Sq, Skv, Hq, D, causal, cus) : 0;
  p.ranges = 1 << l2s;
  p.ws_bytes = split_ws_bytes(B, Sq, Hq, D, p.ranges);
  p.kernel = (l2s > 0 || use_eight_waves(B, Sq, Skv, Hq, D, causal, cus)) ? kEightWave
                                                                          : kFourWave;
  return p;
}

int launch(const LaunchArgs& a) {
  DeviceKernels* dk = nullptr;
  if (kernels_for_current_device(&dk) != hipSuccess) return FA_ERR_HIP;
  const Plan p = make_plan(a.B, a.Sq, a.Skv, a.Hq, a.Hkv, a.D, a.causal, dk->cus, a.ws != nullptr);
  if (p.ranges > 1 && a.ws_bytes < p.ws_bytes) return FA_ERR_WORKSPACE;
  // Split key ranges: the partial results go to the caller's workspace (O
  // [ranges][B][Hq][Sq][D], then LSE [ranges][B][Hq][Sq], fp32) and the
  // combine kernel merges them into o / lse on the same stream.
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (p.ranges > 1) {
    part_o = static_cast<float*>(a.ws);
    part_lse = part_o + (size_t)a.B * a.Hq * a.Sq * p.ranges * a.D;
  }
  hipError_t e;
  if (p.kernel == kTileRows || p.kernel == kTileKeys) {
    e = launch_tile(a, p.kernel == kTileKeys, p.packed, p.ranges, part_o, part_lse);
  } else if (p.ranges > 1) {
    LaunchArgs s = a;
    s.o = part_o;
    s.lse = part_lse;
    int l2s = 0;
    while ((1 << l2s) < p.ranges) ++l2s;
    e = launch_kernel(dk, s, a.dtype == DType::kBF16 ? 6 : 7, true, l2s);
  } else {
    const bool x8 = p.kernel == kEightWave;
    const int variant = x8 ? (a.dtype == DType::kBF16 ? 4 : 5) + (a.D == 128 ? 0 : 4)
                           : (a.dtype == DType::kBF16 ? 0 : 2) + (a.D == 128 ? 0 : 1);
    e = launch_kernel(dk, a, variant, x8, 0);
  }
  if (e == hipSuccess && p.ranges > 1)
    e = launch_combine(a.dtype, part_o, part_lse, a.o, a.lse, p.ranges, a.B, a.Hq, a.Sq, a.D,
                       a.stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

hipError_t launch_kernel(DeviceKernels* dk, const LaunchArgs& a, int variant, bool x8, int l2s) {
  KernArgs ka;
  memset(&ka, 0, sizeof(ka));
  ka.q = a.q;
  ka.k = a.k;
  ka.v = a.v;
  ka.o = a.o;
  ka.lse = a.lse;
  ka.B = a.B;
  ka.Sq = a.Sq;
  ka.Skv = a.Skv;
  ka.Hq = a.Hq;
  ka.Hkv = a.Hkv;
  ka.causal = a.causal;
  ka.c = a.c;
  const int64_t nq = x8 ? ((int64_t)a.Sq + kBM8 - 1) / kBM8 : query_tiles(a.Sq);
  const int64_t items = (nq * a.B * a.Hq) << l2s;
  ka.log2split = (uint32_t)l2s;
  const int64_t grid = items < dk->cus ? items : dk->cus;
  ka.nq_grid = (uint32_t)nq | ((uint32_t)grid << 16);
  if (!group_magic(a.Hq, a.Hkv, &ka.gmagic)) return hipErrorInvalidValue;
  ka.hq_xcd = (a.Hq % 8 == 0) ? (uint32_t)(a.Hq / 8) : 0u;
  size_t size = sizeof(ka);
  void* config[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, &ka, HIP_LAUNCH_PARAM_BUFFER_SIZE, &size,
                    HIP_LAUNCH_PARAM_END};
  // the launch's own status: an earlier, unrelated error left in the
  // runtime's last-error slot is neither reported nor cleared here
  return hipModuleLaunchKernel(dk->fn[variant], (unsigned)grid, 1, 1, x8 ? 512 : 256, 1, 1, 0,
                               a.stream, nullptr, config);
}

}  // namespace fa
