// Bounds model of libtpmlp's kernel launches (test infrastructure, CPU only).
//
// Tiled bf16 GEMM launches are checked lane by lane with the kernel's own
// addressing code (tiled_geometry.hpp): the tile each workgroup takes (the
// XCD-aware order must cover every tile exactly once), the byte range every
// buffer-to-LDS load reads at the first and last k-step it is live (the base
// of a step is affine in k, so those two bound every step between; with a
// split B^T both halves are bounded), that each load's offset stays inside the
// 2 GiB descriptor range unless it is the out-of-range marker, that the loads
// of a stage fill its LDS exactly once, and every epilogue store and read.
// The epilogue's element addresses (row * ld + column, per output) follow the
// kernel's epilogue branches; its rows and columns come from the shared
// coordinate functions.
//
// Every other launch is checked at the level of its arguments: the extents a
// GEMM's arguments imply for each operand (the column map included), and the
// matrices, vectors and workspace slices of the attention, reduction,
// LayerNorm and column-sum launches.
#include "model.hpp"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <set>
#include <string>
#include <vector>

#include "decode_geometry.hpp"
#include "kernels.h"  // from the library's csrc/ (include path)
#include "tiled_geometry.hpp"

namespace hostcheck {
namespace {

struct Buffer {
  uint64_t lo, hi;
  std::string name;
};
std::vector<Buffer> g_bufs;
Stats g_stats;
// Device variables are registered by the library's module constructors, which
// may run before this file's globals are constructed: function-local statics.
std::map<const void *, std::pair<size_t, std::string>> &syms() {
  static std::map<const void *, std::pair<size_t, std::string>> m;
  return m;
}
std::map<const void *, uint64_t> &sym_addr() {
  static std::map<const void *, uint64_t> m;
  return m;
}
std::string g_kernel;  // the launch being checked
int g_launch_findings = 0;

constexpr uint64_t kWindow = uint64_t(1) << 40;  // fake address window per buffer

void finding(const char *fmt, ...) {
  if (g_launch_findings++ >= 4) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_stats.findings.push_back(g_kernel + ": " + buf);
}

// Device variables live as long as the process (the library caches their
// addresses), so their buffers survive reset(), in windows of their own.
std::vector<Buffer> &sym_bufs() {
  static std::vector<Buffer> v;
  return v;
}

const Buffer *find_buf(uint64_t a) {
  for (const Buffer &b : g_bufs)
    if (a >= b.lo && a < b.hi) return &b;
  for (const Buffer &b : sym_bufs())
    if (a >= b.lo && a < b.hi) return &b;
  return nullptr;
}

// [a, a + n) must lie in the buffer that holds `base` (the operand's pointer).
void access(const char *what, uint64_t base, uint64_t a, uint64_t n) {
  ++g_stats.accesses;
  const Buffer *b = find_buf(base);
  if (!b) {
    finding("%s: operand pointer 0x%llx is in no buffer", what, (unsigned long long)base);
    return;
  }
  if (a < b->lo || a + n > b->hi)
    finding("%s: bytes [0x%llx, +%llu) outside %s [0x%llx, 0x%llx)", what,
            (unsigned long long)a, (unsigned long long)n, b->name.c_str(),
            (unsigned long long)b->lo, (unsigned long long)b->hi);
}

// Elements [0, last] of an operand at p (element size es) with `last` the
// largest element index the launch touches; nothing if the range is empty.
void extent(const char *what, const void *p, int64_t last, int es) {
  if (last < 0) return;
  const uint64_t a = (uint64_t)(uintptr_t)p;
  access(what, a, a, (uint64_t)(last + 1) * es);
}

std::vector<int> template_ints(const std::string &name, const char *kernel) {
  std::vector<int> v;
  size_t at = name.find(kernel);
  if (at == std::string::npos) return v;
  at += strlen(kernel);
  if (at >= name.size() || name[at] != 'I') return v;
  ++at;
  // integer (Li<n>E) and bool (Lb<0|1>E) arguments
  while (at + 1 < name.size() && name[at] == 'L' && (name[at + 1] == 'i' || name[at + 1] == 'b')) {
    at += 2;
    const bool neg = name[at] == 'n';
    if (neg) ++at;
    int x = 0;
    while (at < name.size() && name[at] >= '0' && name[at] <= '9') x = 10 * x + (name[at++] - '0');
    v.push_back(neg ? -x : x);
    if (at < name.size() && name[at] == 'E') ++at;
  }
  return v;
}

bool dual_epi(int epi) { return epi == tpmlp::EPI_SWIGLU || epi == tpmlp::EPI_SWIGLU_SAVE; }

int64_t max_src_col(const tpmlp::GemmArgs &p) {
  int64_t m = -1;
  for (int64_t c = 0; c < p.N; ++c) {
    const int64_t s = tpmlp::src_col(p, c);
    if (s > m) m = s;
  }
  return m;
}

// Operand extents implied by a GEMM's arguments (any of the three GEMM
// kernels); es: operand element size (2 for bf16 kernels, 4 for fp32).
void gemm_extents(const tpmlp::GemmArgs &p, int es) {
  using namespace tpmlp;
  if (p.M <= 0 || p.N <= 0 || p.groups <= 0) return;
  const bool dual = dual_epi(p.epi);
  const int64_t mc = max_src_col(p);
  for (int g = 0; g < p.groups; ++g) {
    if (p.lay == LAY_TN)
      extent("A^T", p.A, g * p.sA + (p.K - 1) * p.lda + p.M - 1, es);
    else
      extent("A", p.A, g * p.sA + (p.M - 1) * p.lda + p.K - 1, es);
    if (p.lay == LAY_NT) {
      const int64_t k1 = p.ksplit > 0 ? p.ksplit : p.K;
      extent("B^T", p.B, g * p.sB + mc * p.ldb + k1 - 1, es);
      if (p.ksplit > 0) extent("B2^T", p.B2, mc * p.ldb + (p.K - p.ksplit) - 1, es);
    } else {
      extent("B", p.B, g * p.sB + (p.K - 1) * p.ldb + mc, es);
      if (dual) extent("B2", p.B2, g * p.sB2 + (p.K - 1) * p.ldb2 + mc, es);
    }
    if ((p.epi == EPI_ACT || p.epi == EPI_ACT_SAVE) && p.bias)
      extent("bias", p.bias, g * p.sBias + mc, es);
    const int cw = (p.epi == EPI_DSWIGLU) ? 2 : 1;
    const int ces = (p.epi == EPI_F32 || p.epi == EPI_F32_ACC) ? 4 : es;
    extent("C", p.C, g * p.sC + (p.M - 1) * p.ldc + cw * p.N - 1, ces);
  }
  if (p.epi == EPI_ACT_SAVE) extent("C2", p.C2, (p.M - 1) * p.ldc2 + p.N - 1, es);
  if (p.epi == EPI_SWIGLU_SAVE) extent("C2", p.C2, (p.M - 1) * p.ldc2 + 2 * p.N - 1, es);
  if (p.epi == EPI_DACT) extent("aux", p.aux, (p.M - 1) * p.ldaux + p.N - 1, es);
  if (p.epi == EPI_DSWIGLU) extent("aux", p.aux, (p.M - 1) * p.ldaux + 2 * p.N - 1, es);
}

// ---- the tiled GEMM, lane by lane ------------------------------------------------
// split: the split-K instantiation (S = p.splitk k-ranges per tile, meeting
// in ctr and parts).
template <int BK, int NWAVE, int BM, bool DUAL, int LAY>
void check_tiled(int epi, const tpmlp::GemmArgs &p, unsigned grid, unsigned block, bool split,
                 const unsigned *ctr, const float *parts) {
  using namespace tpmlp;
  using G = tiled::Geom<BK, NWAVE, BM, DUAL, LAY>;
  typedef uint16_t E;  // bf16 storage
  ++g_stats.tiled;
  if (block != (unsigned)(NWAVE * 64)) finding("block %u, want %d", block, NWAVE * 64);
  const int tilesM = (int)((p.M + BM - 1) / BM), tilesN = (int)((p.N + G::NOUT - 1) / G::NOUT);
  const int64_t total = (int64_t)tilesM * tilesN * p.groups;
  const int S = split ? p.splitk : 1;
  if (split && S < 2) finding("split launch with %d k-ranges", S);
  if (S < 1) return;
  if ((int64_t)grid != total * S)
    finding("grid %u, want %lld tiles x %d k-ranges", grid, (long long)total, S);
  const int64_t kc = split ? tiled::split_kc(p.K, S, BK) : p.K;
  if (split) {
    if (kc % BK || (int64_t)S * kc < p.K || (int64_t)(S - 1) * kc >= p.K)
      finding("k-ranges %d x %lld do not tile K %lld", S, (long long)kc, (long long)p.K);
    if (total > (int64_t)kWsMaxBlocks) finding("%lld tiles exceed the counter area", (long long)total);
    // the counters lie in the counter area below the partials
    if ((uint64_t)(uintptr_t)(ctr + total) > (uint64_t)(uintptr_t)parts)
      finding("counters overlap the partials");
    extent("counters", ctr, total - 1, 4);
    extent("partials", parts, total * S * G::SLOT_BYTES / 4 - 1, 4);
    // a slot's groups: a bijection onto its SLOT_BYTES / 16 groups
    std::vector<char> cov((size_t)(G::SLOT_BYTES / 16), 0);
    bool bad = false;
    for (int w = 0; w < NWAVE; ++w)
      for (int lane = 0; lane < 64; ++lane)
        for (int i = 0; i < 4; ++i)
          for (int f = 0; f < G::NB; ++f)
            for (int q = 0; q < 4; ++q) {
              const uint32_t o = G::part_off(w, lane, i, f, q);
              if (o % 16 || o / 16 >= cov.size()) bad = true;
              else if (cov[o / 16]++) bad = true;
            }
    if (bad) finding("partial slot groups are not a bijection");
  }

  // LDS: the loads of all waves fill each stage exactly once, in 1 KiB pieces.
  {
    std::vector<int> cover(G::STAGE_BYTES / 1024, 0);
    bool bad = G::STAGE_BYTES % 1024 != 0;
    for (int w = 0; w < NWAVE; ++w) {
      for (int q = 0; q < G::A_LOADS; ++q) {
        const int o = G::a_lds(w, q);
        if (o < 0 || o + 1024 > G::A_BYTES) bad = true;
        else ++cover[o / 1024];
      }
      for (int j = 0; j < G::B_LOADS; ++j) {
        const int o = G::b_lds(w, j);
        if (o < G::A_BYTES || o + 1024 > G::STAGE_BYTES) bad = true;
        else ++cover[o / 1024];
      }
    }
    for (int c : cover) bad |= c != 1;
    if (bad) finding("stage LDS not filled exactly once");
  }

  std::vector<char> seen((size_t)(total * S), 0);
  const uint64_t Abase = (uint64_t)(uintptr_t)p.A, Bbase = (uint64_t)(uintptr_t)p.B,
                 B2base = (uint64_t)(uintptr_t)p.B2;
  const uint64_t Pb = (uint64_t)(uintptr_t)parts;
  for (unsigned bid = 0; bid < grid; ++bid) {
    int tile = (int)bid, sidx = 0;
    if (split) tiled::split_coords((int)bid, (int)total, tile, sidx);
    int g, tm, tn;
    tiled::tile_coords(tile, tilesM, tilesN, (int)total, g, tm, tn);
    if (g < 0 || g >= p.groups || tm < 0 || tm >= tilesM || tn < 0 || tn >= tilesN || sidx < 0 ||
        sidx >= S) {
      finding("block %u -> tile (%d, %d, %d) range %d out of range", bid, g, tm, tn, sidx);
      continue;
    }
    const int64_t t = ((int64_t)g * tilesM + tm) * tilesN + tn;
    if (seen[t * S + sidx]++) finding("tile (%d, %d, %d) range %d taken twice", g, tm, tn, sidx);
    int64_t kbeg = 0, kend = p.K;
    if (split) tiled::split_range(p.K, kc, sidx, kbeg, kend);
    if (split && kend <= kbeg) finding("empty k-range %d", sidx);
    const int64_t KT = (kend - kbeg + BK - 1) / BK;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * G::NOUT;
    const E *A = G::template a_tile<E>(p, g, m0);
    const E *B = G::template b_group<E>(p, g);
    const E *B2 = G::template b2_group<E>(p, g);
    for (int wave = 0; wave < NWAVE; ++wave) {
      const bool up = G::b_up(wave);
      for (int lane = 0; lane < 64; ++lane) {
        for (int j = 0; j < G::A_LOADS; ++j) {
          uint32_t off;
          int kof;
          G::a_load(p, m0, wave, lane, j, off, kof);
          if (off != tiled::OOB_OFF && off + 16u > 0x7fffffffu)
            finding("A load offset %u past the descriptor range", off);
          // live steps: k0 = kbeg + kt * BK with k0 + kof < kend
          const int64_t last = kend - 1 - kof - kbeg >= 0 ? (kend - 1 - kof - kbeg) / BK : -1;
          for (int64_t kt : {(int64_t)0, last}) {
            if (kt < 0 || kt >= KT) continue;
            const int64_t k0 = kbeg + kt * BK;
            const uint32_t o = G::step_off(kt < KT, k0, kof, kend, off);
            if (o == tiled::OOB_OFF) continue;
            const uint64_t base = (uint64_t)(uintptr_t)G::a_step(p, A, k0);
            access("A load", Abase, base + o, 16);
          }
        }
        for (int j = 0; j < G::B_LOADS; ++j) {
          uint32_t off;
          int kr;
          G::b_load(p, n0, wave, lane, j, off, kr);
          if (off != tiled::OOB_OFF && off + 16u > 0x7fffffffu)
            finding("B load offset %u past the descriptor range", off);
          std::set<int64_t> steps = {0};
          steps.insert(kend - 1 - kr - kbeg >= 0 ? (kend - 1 - kr - kbeg) / BK : -1);
          if (G::TB && p.ksplit > 0) {
            steps.insert((p.ksplit - kbeg) / BK - 1);
            steps.insert((p.ksplit - kbeg) / BK);
          }
          for (int64_t kt : steps) {
            if (kt < 0 || kt >= KT) continue;
            const int64_t k0 = kbeg + kt * BK;
            const uint32_t o = G::step_off(true, k0, kr, kend, off);
            if (o == tiled::OOB_OFF) continue;
            const uint64_t base = (uint64_t)(uintptr_t)G::b_step(p, B, B2, up, k0);
            const bool second = G::TB ? (p.ksplit > 0 && k0 >= p.ksplit) : up;
            access(second ? "B2 load" : "B load", second ? B2base : Bbase, base + o, 16);
          }
        }
      }
    }

    // Split-K: this workgroup's partial slot (stores), every other slot of
    // the tile (the last arriver's loads), the tile's counter.
    if (split) {
      const uint64_t tile0 = Pb + (uint64_t)t * S * G::SLOT_BYTES;
      for (int wave = 0; wave < NWAVE; ++wave)
        for (int lane = 0; lane < 64; ++lane)
          for (int i = 0; i < 4; ++i)
            for (int f = 0; f < G::NB; ++f)
              for (int q = 0; q < 4; ++q) {
                const uint32_t o = G::part_off(wave, lane, i, f, q);
                for (int s2 = 0; s2 < S; ++s2)
                  if (s2 == sidx || (wave == 0 && lane == 0) || (i == 3 && f == G::NB - 1 && q == 3))
                    access(s2 == sidx ? "partial store" : "partial load", Pb,
                           tile0 + (uint64_t)s2 * G::SLOT_BYTES + o, 16);
              }
      if ((int64_t)S * G::SLOT_BYTES > 0x7fffffffLL) finding("slots beyond the descriptor range");
      access("counter", (uint64_t)(uintptr_t)ctr, (uint64_t)(uintptr_t)(ctr + t), 4);
    }

    // Epilogue.  Fragments f of a wave cover its accumulator columns (the
    // gate half's with SwiGLU); rows come in 16 per fragment row block i.
    const int NBO = DUAL ? G::NB / 2 : G::NB;
    const uint64_t Cb = (uint64_t)(uintptr_t)p.C;
    for (int wave = 0; wave < NWAVE; ++wave) {
      const int wm = wave / G::WNW, wn = wave % G::WNW;
      for (int lane = 0; lane < 64; ++lane) {
        const int64_t rbase = G::row_base(m0, wm, lane);
        for (int f = 0; f < NBO; ++f) {
          const int64_t col = G::out_col(n0, wn, f, lane);
          if (col >= p.N) continue;
          if ((epi == EPI_ACT || epi == EPI_ACT_SAVE) && p.bias)
            access("bias", (uint64_t)(uintptr_t)p.bias,
                   (uint64_t)(uintptr_t)p.bias + 2 * (g * p.sBias + src_col(p, col)), 2);
          for (int i = 0; i < 4; ++i) {
            if (epi == EPI_SWIGLU || epi == EPI_ACT) {
              // packed: even lanes store rows of v, odd lanes rows of v + 1,
              // two adjacent columns (col & ~1, +1) as one 4-byte word
              const bool odd = lane & 1;
              const int64_t col0 = col & ~int64_t(1);
              if (col0 + 1 >= p.N) finding("packed store pair at column %lld past N", (long long)col0);
              for (int v = 0; v < 16; v += 2) {
                const int64_t row = G::out_row(rbase, i, v) + (odd ? 1 : 0);
                if (row < p.M)
                  access("C store", Cb, Cb + 2 * (g * p.sC + row * p.ldc + col0), 4);
              }
              continue;
            }
            // the row-max clamp of the epilogues that read before writing
            int64_t rlo = -1;
            for (int v = 0; v < 16; ++v) {
              const int64_t row = G::out_row(rbase, i, v);
              const int64_t r = row < p.M ? row : p.M - 1;
              if (rlo < 0) rlo = r;
              switch (epi) {
                case EPI_F32:
                  if (row < p.M) access("C store", Cb, Cb + 4 * (g * p.sC + row * p.ldc + col), 4);
                  break;
                case EPI_F32_ACC:
                  access("C read", Cb, Cb + 4 * (g * p.sC + r * p.ldc + col), 4);
                  if (row < p.M) access("C store", Cb, Cb + 4 * (g * p.sC + row * p.ldc + col), 4);
                  break;
                case EPI_ACT_SAVE:
                  if (row < p.M) {
                    access("C store", Cb, Cb + 2 * (g * p.sC + row * p.ldc + col), 2);
                    const uint64_t c2 = (uint64_t)(uintptr_t)p.C2;
                    access("C2 store", c2, c2 + 2 * (row * p.ldc2 + col), 2);
                  }
                  break;
                case EPI_SWIGLU_SAVE:
                  if (row < p.M) {
                    access("C store", Cb, Cb + 2 * (g * p.sC + row * p.ldc + col), 2);
                    const uint64_t c2 = (uint64_t)(uintptr_t)p.C2;
                    access("C2 store", c2, c2 + 2 * (row * p.ldc2 + col), 2);
                    access("C2 store", c2, c2 + 2 * (row * p.ldc2 + p.N + col), 2);
                  }
                  break;
                case EPI_DACT:
                case EPI_DSWIGLU: {
                  const uint64_t h = (uint64_t)(uintptr_t)p.aux;
                  const int nh = epi == EPI_DSWIGLU ? 2 : 1;
                  for (int q = 0; q < nh; ++q)
                    access("aux read", h, h + 2 * (r * p.ldaux + q * p.N + col), 2);
                  if (row < p.M) {
                    access("C store", Cb, Cb + 2 * (g * p.sC + row * p.ldc + col), 2);
                    if (epi == EPI_DSWIGLU)
                      access("C store", Cb, Cb + 2 * (g * p.sC + row * p.ldc + p.N + col), 2);
                  }
                  break;
                }
                default:
                  finding("epilogue %d has no model", epi);
                  break;
              }
            }
          }
        }
      }
    }
  }
  for (int64_t t = 0; t < total * S; ++t)
    if (!seen[t]) {
      finding("tile %lld range %lld never taken", (long long)(t / S), (long long)(t % S));
      break;
    }
}

template <int BK, int NWAVE, int BM>
bool dispatch_lay(int epi, int lay, const tpmlp::GemmArgs &p, unsigned grid, unsigned block,
                  bool split, const unsigned *ctr, const float *parts) {
  const bool dual = dual_epi(epi);
  switch (lay * 2 + (dual ? 1 : 0)) {
    case 0: check_tiled<BK, NWAVE, BM, false, 0>(epi, p, grid, block, split, ctr, parts); return true;
    case 1: check_tiled<BK, NWAVE, BM, true, 0>(epi, p, grid, block, split, ctr, parts); return true;
    case 2: check_tiled<BK, NWAVE, BM, false, 1>(epi, p, grid, block, split, ctr, parts); return true;
    case 4: check_tiled<BK, NWAVE, BM, false, 2>(epi, p, grid, block, split, ctr, parts); return true;
  }
  return false;
}

void on_tiled(const std::vector<int> &t, void **args, unsigned grid, unsigned block) {
  // <EPI, ACT, BK, NST, NWAVE, BM, LAY, SPLIT>(GemmArgs, ctr, parts)
  const tpmlp::GemmArgs &p = *(const tpmlp::GemmArgs *)args[0];
  const unsigned *ctr = *(unsigned *const *)args[1];
  const float *parts = *(float *const *)args[2];
  if (t.size() != 8) {
    finding("cannot read the template arguments");
    return;
  }
  const int epi = t[0], BK = t[2], NWAVE = t[4], BM = t[5], LAY = t[6];
  const bool split = t[7] != 0;
  if (epi != p.epi || LAY != p.lay) finding("kernel <epi %d, lay %d> launched with args epi %d lay %d", epi, LAY, p.epi, p.lay);
  if (!split && (ctr || parts)) finding("unsplit launch given a workspace");
  gemm_extents(p, 2);
  bool ok = false;
  if (BK == 32 && NWAVE == 8 && BM == 256) ok = dispatch_lay<32, 8, 256>(epi, LAY, p, grid, block, split, ctr, parts);
  else if (BK == 32 && NWAVE == 4 && BM == 256) ok = dispatch_lay<32, 4, 256>(epi, LAY, p, grid, block, split, ctr, parts);
  else if (BK == 32 && NWAVE == 4 && BM == 128) ok = dispatch_lay<32, 4, 128>(epi, LAY, p, grid, block, split, ctr, parts);
  else if (BK == 32 && NWAVE == 8 && BM == 128) ok = dispatch_lay<32, 8, 128>(epi, LAY, p, grid, block, split, ctr, parts);
  else if (BK == 64 && NWAVE == 8 && BM == 256) ok = dispatch_lay<64, 8, 256>(epi, LAY, p, grid, block, split, ctr, parts);
  if (!ok) finding("no model for tile configuration BK %d NWAVE %d BM %d", BK, NWAVE, BM);
}

// ---- the few-token GEMM, lane by lane ---------------------------------------------
template <int MB, int BK, int NST>
void check_decode(int epi, const tpmlp::GemmArgs &p, int64_t nblk, int64_t S, int64_t kc,
                  const unsigned *ctr, const float *parts, unsigned grid, unsigned block) {
  using namespace tpmlp;
  using G = decode::Geo<MB, BK, NST>;
  const int nmat = epi == EPI_SWIGLU ? 2 : 1;
  const int64_t nparts = nmat * S;
  if (block != (unsigned)(decode::NWAVE * 64)) finding("block %u", block);
  // LDS: every stage's weight region and token region filled exactly once.
  {
    std::vector<int> cover(G::SB, 0);
    bool bad = false;
    for (int w = 0; w < decode::NWAVE; ++w) {
      for (int j = 0; j < G::WL; ++j) {
        const int o = G::w_lds(w, j);
        if (o < 0 || o + 1024 > G::WB) bad = true;
        else for (int b = 0; b < 1024; ++b) ++cover[o + b];
      }
      for (int j = 0; j < G::XL; ++j) {
        const int o = G::x_lds(w, j);
        for (int lane = 0; lane < 64; ++lane) {
          if (!G::x_lane(lane)) continue;
          const int b0 = o + lane * G::X_BYTES;
          if (b0 < G::WB || b0 + G::X_BYTES > G::SB) bad = true;
          else for (int b = 0; b < G::X_BYTES; ++b) ++cover[b0 + b];
        }
      }
    }
    for (int c : cover) bad |= c != 1;
    if (bad) finding("stage LDS not filled exactly once");
  }
  std::vector<char> seen((size_t)(nblk * nmat * S), 0);
  const uint64_t Xb = (uint64_t)(uintptr_t)p.A, Cb = (uint64_t)(uintptr_t)p.C;
  const uint64_t Pb = (uint64_t)(uintptr_t)parts;
  std::vector<std::pair<uint64_t, unsigned>> pstores;  // (16-byte group, workgroup)
  for (unsigned bid = 0; bid < grid; ++bid) {
    int64_t blk, s, kbeg, kend;
    bool up;
    decode::wg_coords(bid, nmat, nblk, blk, s, up);
    if (blk < 0 || blk >= nblk || s < 0 || s >= S) {
      finding("workgroup %u -> block %lld range %lld out of range", bid, (long long)blk, (long long)s);
      continue;
    }
    const int64_t u = (s * nmat + (up ? 1 : 0)) * nblk + blk;
    if (seen[u]++) finding("block %lld range %lld taken twice", (long long)blk, (long long)s);
    decode::k_range(s, kc, p.K, kbeg, kend);
    if (kend <= kbeg) finding("empty k-range %lld", (long long)s);
    const int64_t nst = (kend - kbeg + BK - 1) / BK;
    const uint64_t Wb = (uint64_t)(uintptr_t)(up ? p.B2 : p.B);
    const int64_t ldw = up ? p.ldb2 : p.ldb;
    const int64_t n0 = blk * decode::RC;
    // the stages a load with relative k `k` is live in: first and last
    auto stages = [&](int k, int64_t &t0, int64_t &t1) {
      t0 = 0;
      t1 = kend - 1 - kbeg - k >= 0 ? (kend - 1 - kbeg - k) / BK : -1;
      if (t1 > nst - 1) t1 = nst - 1;
    };
    for (int wave = 0; wave < decode::NWAVE; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        for (int j = 0; j < G::WL; ++j) {
          uint32_t off;
          int row;
          G::w_load(p, ldw, n0, wave, lane, j, off, row);
          if (off != decode::OOB_OFF && off + 16u > 0x7fffffffu) finding("weight offset %u", off);
          int64_t t0, t1;
          stages(row, t0, t1);
          for (int64_t t : {t0, t1}) {
            if (t < 0 || t > t1) continue;
            const int64_t k0 = kbeg + t * BK;
            const uint32_t o = G::stage_off(true, k0, row, kend, off);
            if (o != decode::OOB_OFF) access(up ? "Wu load" : "W load", Wb, Wb + 2 * k0 * ldw + o, 16);
          }
        }
        for (int j = 0; j < G::XL; ++j) {
          if (!G::x_lane(lane)) continue;
          uint32_t off;
          int k;
          G::x_load(p, wave, lane, j, off, k);
          if (off != decode::OOB_OFF && off + 16u > 0x7fffffffu) finding("token offset %u", off);
          int64_t t0, t1;
          stages(k, t0, t1);
          for (int64_t t : {t0, t1}) {
            if (t < 0 || t > t1) continue;
            const int64_t k0 = kbeg + t * BK;
            const uint32_t o = G::stage_off(true, k0, k, kend, off);
            if (o != decode::OOB_OFF) access("X load", Xb, Xb + 2 * k0 + o, G::X_BYTES);
          }
        }
        const int64_t col = decode::out_col(n0, wave, lane);
        if (nparts > 1) {
          const uint64_t blk0 = Pb + 4 * (uint64_t)(blk * G::block_floats(nparts));
          for (int m = 0; m < MB; ++m) {
            const uint32_t g = G::group_off(p.M, wave, lane, m);
            if (g == decode::OOB_OFF) continue;
            access("partial store", Pb, blk0 + g + G::slot_off(up ? 1 : 0, S, s), 16);
            pstores.emplace_back(blk0 + g + G::slot_off(up ? 1 : 0, S, s), bid);
            for (int q = 0; q < nmat; ++q)
              for (int64_t s2 = 0; s2 < S; ++s2)
                access("partial load", Pb, blk0 + g + G::slot_off(q, S, s2), 16);
          }
          if (wave == 0 && lane == 0)
            access("counter", (uint64_t)(uintptr_t)ctr, (uint64_t)(uintptr_t)(ctr + blk), 4);
        }
        // the output: written by the block's only workgroup, or its last arriver
        if (col < p.N && (nparts > 1 || !up)) {
          if (epi == EPI_ACT && p.bias)
            access("bias", (uint64_t)(uintptr_t)p.bias,
                   (uint64_t)(uintptr_t)p.bias + 2 * src_col(p, col), 2);
          const int es = epi == EPI_F32 ? 4 : 2;
          for (int m = 0; m < MB; ++m)
            for (int v = 0; v < 4; ++v) {
              const int64_t row = decode::out_row(m, lane, v);
              if (row < p.M) access("C store", Cb, Cb + es * (row * p.ldc + col), es);
            }
        }
      }
  }
  for (size_t u = 0; u < seen.size(); ++u)
    if (!seen[u]) {
      finding("work item %zu never taken", u);
      break;
    }
  // No two workgroups' partial stores may overlap (16-byte aligned groups).
  std::sort(pstores.begin(), pstores.end());
  for (size_t i = 1; i < pstores.size(); ++i)
    if (pstores[i].first < pstores[i - 1].first + 16 && pstores[i].second != pstores[i - 1].second) {
      finding("partial stores of workgroups %u and %u overlap", pstores[i - 1].second,
              pstores[i].second);
      break;
    }
}

// ---- argument-level models of the other kernels ------------------------------------
void on_decode(const std::vector<int> &t, void **args, unsigned grid, unsigned block) {
  // <EPI, ACT, MB, BK, NST>(GemmArgs, nblk, S, kc, ctr, parts)
  const tpmlp::GemmArgs &p = *(const tpmlp::GemmArgs *)args[0];
  const int64_t nblk = *(const int64_t *)args[1], S = *(const int64_t *)args[2],
                kc = *(const int64_t *)args[3];
  const unsigned *ctr = *(unsigned *const *)args[4];
  const float *parts = *(float *const *)args[5];
  if (t.size() != 5) {
    finding("cannot read the template arguments");
    return;
  }
  const int MB = t[2], BK = t[3], NST = t[4];
  const int nmat = t[0] == tpmlp::EPI_SWIGLU ? 2 : 1;
  const int nwave = (int)block / 64;
  gemm_extents(p, 2);
  if (p.M > 16 * MB) finding("M %lld above the %d token rows of the configuration", (long long)p.M, 16 * MB);
  if ((int64_t)grid != nblk * nmat * S) finding("grid %u, want %lld", grid, (long long)(nblk * nmat * S));
  if (nblk * 16 * nwave < p.N) finding("column blocks cover %lld of %lld", (long long)(nblk * 16 * nwave), (long long)p.N);
  if (S * kc < p.K || (S - 1) * kc >= p.K) finding("k-ranges %lld x %lld do not tile K %lld", (long long)S, (long long)kc, (long long)p.K);
  if (nmat * S > 1) {
    extent("counters", ctr, nblk - 1, 4);
    extent("partials", parts, nblk * nmat * S * (int64_t)nwave * MB * 256 - 1, 4);
  }
  ++g_stats.decode;
  if (MB == 1 && BK == 32 && NST == 4)
    check_decode<1, 32, 4>(t[0], p, nblk, S, kc, ctr, parts, grid, block);
  else if (MB == 2 && BK == 32 && NST == 4)
    check_decode<2, 32, 4>(t[0], p, nblk, S, kc, ctr, parts, grid, block);
  else if (MB == 4 && BK == 64 && NST == 3)
    check_decode<4, 64, 3>(t[0], p, nblk, S, kc, ctr, parts, grid, block);
  else
    finding("no model for configuration MB %d BK %d NST %d", MB, BK, NST);
}

void on_f32(const tpmlp::GemmArgs &p) { gemm_extents(p, 4); }

void on_attention(void **args) {
  const tpmlp::AttnArgs &a = *(const tpmlp::AttnArgs *)args[0];
  const int64_t T = a.nseq * a.S;
  extent("Q", a.Q, (T - 1) * a.ldq + (int64_t)a.Hq * a.dh - 1, 2);
  extent("K", a.K, (T - 1) * a.ldk + (int64_t)a.Hkv * a.dh - 1, 2);
  extent("V", a.V, (T - 1) * a.ldv + (int64_t)a.Hkv * a.dh - 1, 2);
  extent("O", a.O, (T - 1) * a.ldo + (int64_t)a.Hq * a.dh - 1, 2);
}

void on_partial_sum(void **args) {
  const tpmlp::PartSumArgs &a = *(const tpmlp::PartSumArgs *)args[0];
  for (int j = 0; j < a.p; ++j) extent("part", a.parts[j], (a.T - 1) * a.ldp + a.d - 1, 4);
  if (a.b2) extent("b2", a.b2, a.d - 1, 4);
  extent("Z", a.Z, (a.T - 1) * a.ldz + a.d - 1, 4);
}

void on_residual_ln(void **args) {
  const tpmlp::RowNormArgs &a = *(const tpmlp::RowNormArgs *)args[0];
  for (int j = 0; j < a.p; ++j) extent("part", a.parts[j], (a.T - 1) * a.ldp + a.d - 1, 4);
  if (a.bias) extent("bias", a.bias, a.d - 1, 4);
  if (a.R) extent("R", a.R, (a.T - 1) * a.ldr + a.d - 1, 4);
  if (a.X) extent("X", a.X, (a.T - 1) * a.ldx + a.d - 1, 4);
  if (a.gamma) {
    extent("gamma", a.gamma, a.d - 1, 4);
    extent("beta", a.beta, a.d - 1, 4);
    extent("A", a.A, (a.T - 1) * a.lda + a.d - 1, 2);
  }
}

void on_colsum(bool chunks, bool bf16_in, void **args, unsigned gy) {
  if (chunks) {  // (H, ldh, T, n, ws)
    const void *H = *(const void *const *)args[0];
    const int64_t ldh = *(const int64_t *)args[1], T = *(const int64_t *)args[2],
                  n = *(const int64_t *)args[3];
    const float *ws = *(float *const *)args[4];
    extent("H", H, (T - 1) * ldh + n - 1, bf16_in ? 2 : 4);
    extent("colsum scratch", ws, (int64_t)gy * n - 1, 4);
  } else {  // (part, chunks, n, out)
    const float *part = *(float *const *)args[0];
    const int64_t ch = *(const int64_t *)args[1], n = *(const int64_t *)args[2];
    const float *out = *(float *const *)args[3];
    extent("colsum scratch", part, ch * n - 1, 4);
    extent("column sums", out, n - 1, 4);
  }
}

}  // namespace

void *fake_alloc(size_t bytes, const char *name) {
  const uint64_t lo = kWindow * (g_bufs.size() + 1);
  g_bufs.push_back(Buffer{lo, lo + bytes, name});
  return (void *)(uintptr_t)lo;
}

void reset() {
  g_bufs.clear();
  g_stats = Stats();
}

Stats &stats() { return g_stats; }

void register_symbol(const void *host_var, size_t bytes, const char *name) {
  syms()[host_var] = {bytes, name ? name : "symbol"};
}

void *symbol_address(const void *host_var) {
  auto it = syms().find(host_var);
  if (it == syms().end()) return nullptr;
  auto a = sym_addr().find(host_var);
  if (a == sym_addr().end()) {
    const uint64_t lo = kWindow * (4096 + sym_bufs().size());
    sym_bufs().push_back(Buffer{lo, lo + it->second.first, it->second.second});
    a = sym_addr().emplace(host_var, lo).first;
  }
  return (void *)(uintptr_t)a->second;
}

void on_launch(const char *name, unsigned gx, unsigned gy, unsigned gz, unsigned bx, unsigned by,
               unsigned bz, void **args) {
  const std::string n(name);
  g_kernel = n;
  g_launch_findings = 0;
  ++g_stats.launches;
  g_stats.kernels.push_back(n);
  if (by != 1 || bz != 1) finding("block is not one-dimensional");
  if (n.find("gemm_bf16_tiled_kernel") != std::string::npos) {
    if (gy != 1 || gz != 1) finding("grid is not one-dimensional");
    on_tiled(template_ints(n, "gemm_bf16_tiled_kernel"), args, gx, bx);
    return;
  }
  ++g_stats.checked_other;
  if (n.find("gemm_bf16_decode_kernel") != std::string::npos)
    on_decode(template_ints(n, "gemm_bf16_decode_kernel"), args, gx, bx);
  else if (n.find("gemm_f32_kernel") != std::string::npos)
    on_f32(*(const tpmlp::GemmArgs *)args[0]);
  else if (n.find("attention_kernel") != std::string::npos)
    on_attention(args);
  else if (n.find("partial_sum_kernel") != std::string::npos)
    on_partial_sum(args);
  else if (n.find("residual_ln_kernel") != std::string::npos)
    on_residual_ln(args);
  else if (n.find("colsum_chunks") != std::string::npos)
    on_colsum(true, n.find("colsum_chunksI") != std::string::npos &&
                        n.find("DF16b") != std::string::npos,
              args, gy);
  else if (n.find("colsum_final") != std::string::npos)
    on_colsum(false, false, args, gy);
  else
    --g_stats.checked_other;  // zero-fill and measurement kernels: recorded only
}

}  // namespace hostcheck
