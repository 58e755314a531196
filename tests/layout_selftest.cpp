// Host-side check of the kernel's index arithmetic (fa_layout.h), built with g++.
//
// It simulates, for one wave, the gfx950 data movement the kernel relies on --
// the direct-to-LDS tile copy, the 16-byte fragment reads, the transposing
// ds_read_b64_tr_b16 reads and the MFMA 32x32x16 operand/accumulator layouts --
// using the lane semantics stated in fa_layout.h, and checks that every MFMA
// operand element is the tensor element the math needs. Exit code 0 = pass.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

#include "fa_layout.h"

static int g_fail = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      if (g_fail < 20) {                 \
        std::printf("FAIL: " __VA_ARGS__); \
        std::printf("\n");               \
      }                                  \
      ++g_fail;                          \
    }                                    \
  } while (0)

// An LDS tile image: for every 16-bit slot, the (row, col) of the tensor element stored there.
struct Elt {
  int row, col;
};

template <int D, int ROWS, bool TR>
std::vector<Elt> dma_image() {
  const int n_inst = fa::dma_insts<D, ROWS>();
  std::vector<Elt> lds(ROWS * D, Elt{-1, -1});
  std::set<std::pair<int, int>> seen;
  const int64_t stride = 1000 * 16;  // any row stride: checks the lane/instruction split of the source
  for (int inst = 0; inst < n_inst; ++inst)
    for (int lane = 0; lane < 64; ++lane) {
      fa::RowChunk rc = fa::dma_source<D, ROWS, TR>(inst, lane);
      CHECK(rc.row >= 0 && rc.row < ROWS && rc.chunk >= 0 && rc.chunk < D / 8, "dma source out of tile D=%d", D);
      CHECK(seen.insert({rc.row, rc.chunk}).second, "dma copies a chunk twice D=%d", D);
      const int byte = inst * 1024 + lane * 16;  // where the direct-to-LDS load puts this lane's 16 bytes
      CHECK(byte == (fa::tile_chunk_offset<D, ROWS, TR>(rc.row, rc.chunk)), "dma slot != tile_chunk_offset D=%d", D);
      const int64_t src = fa::dma_lane_offset<D, TR>(lane, stride) + fa::dma_inst_offset<D, ROWS>(inst, stride);
      CHECK(src == rc.row * stride + rc.chunk * 16, "dma source offset split D=%d", D);
      for (int e = 0; e < 8; ++e) lds[byte / 2 + e] = Elt{rc.row, rc.chunk * 8 + e};
    }
  CHECK((int)seen.size() == ROWS * D / 8, "dma misses chunks D=%d", D);
  return lds;
}

template <int D>
void check_d() {
  constexpr int BKV = 64;
  std::vector<Elt> lds = dma_image<D, BKV, false>();
  std::vector<Elt> vlds = dma_image<D, BKV, true>();
  const int NS = D / 16;
  // K fragment (A operand of S^T = K Q^T): lane l must hold K[32kb + l%32][16s + 8(l/32) + e]
  for (int kb = 0; kb < BKV / 32; ++kb)
    for (int s = 0; s < NS; ++s)
      for (int lane = 0; lane < 64; ++lane) {
        const int byte = fa::tile_chunk_offset<D, BKV, false>(fa::kfrag_row(kb, lane), fa::kfrag_chunk(s, lane));
        const int split = fa::kfrag_lane_offset<D, BKV>(s % fa::kfrag_parities<D>(), lane) +
                          fa::kfrag_const_offset<D, BKV>(kb, s);
        CHECK(byte == split, "K offset split D=%d", D);
        for (int e = 0; e < 8; ++e) {
          const Elt x = lds[byte / 2 + e];
          CHECK(x.row == 32 * kb + lane % 32 && x.col == 16 * s + 8 * (lane / 32) + e, "K frag D=%d", D);
        }
      }
  // V^T fragment (A operand of O^T = V^T P^T) via two transposing reads; lane l must hold
  // V[key(ks, l, e)][32db + l%32] for e = 0..7 (lanes with l%32 >= D hold padding).
  const int NDB = D < 32 ? 1 : D / 32;
  for (int db = 0; db < NDB; ++db)
    for (int ks = 0; ks < BKV / 16; ++ks)
      for (int half = 0; half < 2; ++half) {
        int addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          addr[lane] = fa::tile_quad_offset<D, BKV>(fa::vtr_row(ks, half, lane), fa::vtr_col_clamped<D>(db, lane));
          const int split = fa::vtr_lane_offset<D, BKV>(lane) + fa::vtr_const_offset<D, BKV>(ks, half, db);
          CHECK(addr[lane] == split, "V offset split D=%d", D);
          CHECK(addr[lane] % 8 == 0 && addr[lane] >= 0 && addr[lane] + 8 <= BKV * D * 2, "tr addr D=%d", D);
        }
        for (int lane = 0; lane < 64; ++lane) {
          if (D < 32 && ((lane >> 4) & 1)) continue;  // padding lanes are zeroed by the kernel
          for (int e = 0; e < 4; ++e) {
            const int src = 16 * (lane / 16) + 4 * e + (lane % 16) / 4;
            const Elt x = vlds[addr[src] / 2 + (lane % 4)];
            const int ee = 4 * half + e;
            CHECK(x.row == fa::pv_key(ks, lane, ee) && x.col == 32 * db + lane % 32, "V^T frag D=%d", D);
          }
        }
        // bank behaviour: each 16-lane group touches 8 chunks on 8 distinct 16-byte slots of the
        // 256-byte bank line, each 32-lane half 16 distinct slots (D >= 32)
        for (int span = 16; span <= (D >= 32 ? 32 : 16); span *= 2)
          for (int g0 = 0; g0 < 64; g0 += span) {
            std::set<int> slots, chunks;
            for (int lane = g0; lane < g0 + span; ++lane) {
              chunks.insert(addr[lane] / 16);
              slots.insert((addr[lane] / 16) % 16);
            }
            CHECK(slots.size() == chunks.size(), "V tr read bank conflict D=%d span=%d", D, span);
          }
      }
  // bank behaviour of the 16-byte fragment reads: the 16 lanes of a phase hit 16 distinct slots
  for (int kb = 0; kb < BKV / 32; ++kb)
    for (int s = 0; s < NS; ++s)
      for (int ph = 0; ph < 4; ++ph) {
        std::set<int> slots;
        for (int lane = 16 * ph; lane < 16 * ph + 16; ++lane)
          slots.insert((fa::tile_chunk_offset<D, BKV, false>(fa::kfrag_row(kb, lane), fa::kfrag_chunk(s, lane)) / 16) % 16);
        CHECK(slots.size() == 16, "K read bank conflict D=%d", D);
      }
}

// Transposing reads of a swizzled tile (read as row fragments as well): the same operand elements
// as from the unswizzled layout, and no bank conflicts for either kind of read.
template <int D, int ROWS>
void check_swizzled_transpose() {
  std::vector<Elt> lds = dma_image<D, ROWS, false>();
  const int NDB = D < 32 ? 1 : D / 32;
  for (int db = 0; db < NDB; ++db)
    for (int ks = 0; ks < ROWS / 16; ++ks)
      for (int half = 0; half < 2; ++half) {
        int addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          const int row = fa::vtr_row(ks, half, lane), col = fa::vtr_col_clamped<D>(db, lane);
          addr[lane] = fa::tile_chunk_offset<D, ROWS, false>(row, col / 8) + (col % 8) * 2;
          const int split = fa::vtr_swz_lane_offset<D, ROWS>(half, lane) + fa::vtr_swz_const_offset<D, ROWS>(ks, db);
          CHECK(addr[lane] == split, "swizzled tr offset split D=%d ROWS=%d", D, ROWS);
          CHECK(addr[lane] % 8 == 0 && addr[lane] >= 0 && addr[lane] + 8 <= ROWS * D * 2, "swizzled tr addr D=%d", D);
        }
        for (int lane = 0; lane < 64; ++lane) {
          if (D < 32 && ((lane >> 4) & 1)) continue;  // padding lanes are zeroed by the kernel
          for (int e = 0; e < 4; ++e) {
            const int src = 16 * (lane / 16) + 4 * e + (lane % 16) / 4;
            const Elt x = lds[addr[src] / 2 + (lane % 4)];
            CHECK(x.row == fa::pv_key(ks, lane, 4 * half + e) && x.col == 32 * db + lane % 32,
                  "swizzled tr operand D=%d ROWS=%d", D, ROWS);
          }
        }
        for (int span = 16; span <= (D >= 32 ? 32 : 16); span *= 2)
          for (int g0 = 0; g0 < 64; g0 += span) {
            std::set<int> slots, chunks;
            for (int lane = g0; lane < g0 + span; ++lane) {
              chunks.insert(addr[lane] / 16);
              slots.insert((addr[lane] / 16) % 16);
            }
            CHECK(slots.size() == chunks.size(), "swizzled tr read bank conflict D=%d ROWS=%d span=%d", D, ROWS, span);
          }
      }
  // and its row fragments through the swizzled fragment offsets
  for (int kb = 0; kb < ROWS / 32; ++kb)
    for (int s = 0; s < D / 16; ++s) {
      for (int lane = 0; lane < 64; ++lane) {
        const int byte = fa::kfrag_lane_offset<D, ROWS>(s % fa::kfrag_parities<D>(), lane) +
                         fa::kfrag_const_offset<D, ROWS>(kb, s);
        for (int e = 0; e < 8; ++e) {
          const Elt x = lds[byte / 2 + e];
          CHECK(x.row == 32 * kb + lane % 32 && x.col == 16 * s + 8 * (lane / 32) + e, "row frag D=%d ROWS=%d", D, ROWS);
        }
      }
      for (int ph = 0; ph < 4; ++ph) {
        std::set<int> slots;
        for (int lane = 16 * ph; lane < 16 * ph + 16; ++lane)
          slots.insert(((fa::kfrag_lane_offset<D, ROWS>(s % fa::kfrag_parities<D>(), lane) +
                         fa::kfrag_const_offset<D, ROWS>(kb, s)) / 16) % 16);
        CHECK(slots.size() == 16, "row frag bank conflict D=%d ROWS=%d", D, ROWS);
      }
    }
}

int main() {
  check_swizzled_transpose<16, 64>();
  check_swizzled_transpose<32, 64>();
  check_swizzled_transpose<64, 64>();
  check_swizzled_transpose<128, 64>();
  check_swizzled_transpose<256, 64>();
  check_swizzled_transpose<256, 32>();
  check_swizzled_transpose<128, 32>();
  check_d<16>();
  check_d<32>();
  check_d<64>();
  check_d<128>();
  check_d<256>();
  // P^T operand taken from the S^T accumulators: register pv_src_reg(ks, e) of key block ks/2
  for (int ks = 0; ks < 4; ++ks)
    for (int lane = 0; lane < 64; ++lane)
      for (int e = 0; e < 8; ++e) {
        const int key = 32 * (ks / 2) + fa::acc_row(fa::pv_src_reg(ks, e), lane);
        CHECK(key == fa::pv_key(ks, lane, e), "P operand key");
      }
  // pv_key is a bijection of the 16 keys of a slice onto operand positions
  for (int ks = 0; ks < 2; ++ks) {
    std::set<int> keys;
    for (int lane = 0; lane < 64; lane += 32)
      for (int e = 0; e < 8; ++e) keys.insert(fa::pv_key(ks, lane, e));
    CHECK((int)keys.size() == 16 && *keys.begin() == 16 * ks && *keys.rbegin() == 16 * ks + 15, "pv_key perm");
  }
  // the work schedule visits every (batch, head, query tile) exactly once, keeps each whole unit on
  // one XCD and each leftover unit with its own share on at most that share, and (causal) lists the
  // items run at once longest first, or else the leftover items longest first and then each whole
  // unit's items together, longest first
  for (int B : {1, 2, 3, 4, 5, 9, 13})
    for (int hkv : {1, 2, 3, 8, 16})
      for (int group : {1, 3, 4})
        for (int n_qt : {1, 3, 8, 17})
          for (int causal = 0; causal < 2; ++causal)
            for (int grid : {1, 5, 64, 256, 512, 768, 1024}) {
              fa::Schedule sc{B * hkv, hkv, group, n_qt, causal != 0, 0};
              const long n_items = (long)B * hkv * group * n_qt;
              sc.grid = sc.choose_grid(grid);
              CHECK(sc.grid >= 1 && (sc.grid >= 8 || sc.grid >= n_items), "grid leaves an XCD without workgroups");
              long total = 0;
              for (int x = 0; x < 8; ++x) {
                total += sc.items_of(x);
                CHECK(sc.items_of(x) == 0 || sc.wgs_of(x) > 0, "an XCD holds items but no workgroup");
              }
              CHECK(total == n_items, "items per XCD do not add up");
              std::vector<int> seen(n_items, 0);
              std::map<int, std::set<int>> unit_xcds;
              for (int wg = 0; wg < sc.grid; ++wg) {
                const int x = wg % 8;
                for (long r = 0;; ++r) {
                  const long i = sc.item_index(wg, r);
                  if (i >= sc.items_of(x)) break;
                  const fa::Item it = sc.item(x, i);
                  CHECK(it.b >= 0 && it.b < B && it.h >= 0 && it.h < hkv * group && it.qt >= 0 && it.qt < n_qt,
                        "schedule item out of range");
                  if (!(it.b >= 0 && it.b < B && it.h >= 0 && it.h < hkv * group && it.qt >= 0 && it.qt < n_qt)) break;
                  seen[((long)it.b * hkv * group + it.h) * n_qt + it.qt]++;
                  unit_xcds[it.b * hkv + it.h / group].insert(x);
                }
              }
              for (long k = 0; k < n_items; ++k) CHECK(seen[k] == 1, "schedule misses or repeats an item");
              for (auto& kv : unit_xcds) {
                if (kv.first < 8 * sc.whole())
                  CHECK(kv.second.size() == 1 && *kv.second.begin() == kv.first % 8, "whole unit not on its XCD");
                else if (sc.shared_rest())
                  CHECK((int)kv.second.size() <= sc.share(), "leftover unit spread beyond its share");
              }
              if (causal)
                for (int x = 0; x < 8; ++x) {
                  if (sc.one_round(x)) {
                    for (long i = 1; i < sc.items_of(x); ++i)
                      CHECK(sc.item(x, i).qt <= sc.item(x, i - 1).qt, "causal items of one round not longest first");
                    continue;
                  }
                  const long nl = sc.left_of(x);
                  std::set<int> done;
                  for (long i = 1; i < sc.items_of(x); ++i) {
                    const fa::Item a = sc.item(x, i - 1), c = sc.item(x, i);
                    const int ua = a.b * hkv + a.h / group, uc = c.b * hkv + c.h / group;
                    if (i < nl) {
                      CHECK(c.qt <= a.qt, "leftover items not longest first");
                      continue;
                    }
                    if (i == nl) continue;  // first whole-unit item
                    if (ua == uc)
                      CHECK(c.qt <= a.qt, "causal items of a unit not longest first");
                    else
                      CHECK(done.insert(ua).second && !done.count(uc), "a unit's items are not listed together");
                  }
                }
            }
  // balance across the XCDs for any number of (batch, kv head) units: with at least four items per
  // XCD, the most loaded XCD holds at most 10 % more items, and (causal) 10 % more key tiles, than
  // the mean
  for (int n_units = 1; n_units <= 64; ++n_units)
    for (int group : {1, 3, 4})
      for (int n_qt : {8, 16, 32, 128})
        for (int causal = 0; causal < 2; ++causal) {
          if ((long)n_units * group * n_qt < 32) continue;
          fa::Schedule sc{n_units, 1, group, n_qt, causal != 0, 0};
          sc.grid = sc.choose_grid(512);
          double cnt[8] = {0}, work[8] = {0}, mc = 0, mw = 0, xc = 0, xw = 0;
          for (int x = 0; x < 8; ++x)
            for (long i = 0; i < sc.items_of(x); ++i) {
              cnt[x] += 1;
              work[x] += causal ? sc.item(x, i).qt + 1 : n_qt;
            }
          for (int x = 0; x < 8; ++x) {
            mc += cnt[x] / 8;
            mw += work[x] / 8;
            xc = xc > cnt[x] ? xc : cnt[x];
            xw = xw > work[x] ? xw : work[x];
          }
          CHECK(xc <= 1.1 * mc && xw <= 1.1 * mw, "XCD imbalance: %d units, group %d, %d query tiles, causal %d: "
                "items %.0f / %.2f, work %.0f / %.2f", n_units, group, n_qt, causal, xc, mc, xw, mw);
        }
  // causal balance of the workload of 4 batches x 16 heads x 8 query tiles (2..16 key tiles each)
  // on 2 resident workgroups per CU: every CU gets the same total
  {
    fa::Schedule sc{64, 16, 1, 8, true, 0};
    sc.grid = sc.choose_grid(512);
    std::map<std::pair<int, int>, int> cu_load;
    for (int wg = 0; wg < sc.grid; ++wg) {
      const int x = wg % 8, k = wg / 8;
      for (long r = 0;; ++r) {
        const long i = sc.item_index(wg, r);
        if (i >= sc.items_of(x)) break;
        cu_load[{x, k % fa::kCUsPerXCD}] += 2 * (sc.item(x, i).qt + 1);
      }
    }
    for (auto& kv : cu_load) CHECK(kv.second == 18, "unbalanced CU: %d key tiles", kv.second);
  }
  // key tiles per query tile against a brute-force scan of the visible (row, key) pairs
  for (int nq : {1, 7, 64, 100, 128, 300})
    for (int nkv : {1, 5, 64, 130, 257})
      for (int bq : {32, 128})
        for (int bkv : {32, 64})
          for (int causal = 0; causal < 2; ++causal)
            for (int q0 = 0; q0 < nq; q0 += bq) {
              int need = 0;
              for (int i = q0; i < q0 + bq && i < nq; ++i)
                for (int j = 0; j < nkv; ++j)
                  if (!causal || j <= i) need = need > j / bkv + 1 ? need : j / bkv + 1;
              const long got = fa::kv_tiles_for_qtile(q0, bq, nkv, bkv, causal);
              // the kernel may visit a tile that only rows past nq would see (they are never stored)
              CHECK(got >= need && got <= (nkv + bkv - 1) / bkv, "kv tiles nq=%d nkv=%d", nq, nkv);
              if (q0 + bq <= nq) CHECK(got == need, "kv tiles exact nq=%d nkv=%d", nq, nkv);
            }
  if (g_fail) {
    std::printf("%d layout checks failed\n", g_fail);
    return 1;
  }
  std::printf("layout self-test passed\n");
  return 0;
}
