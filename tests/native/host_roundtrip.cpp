// Host-side round trip of the packed image under AddressSanitizer and UBSan:
// the library's encoder, packer and unpacker (no GPU code) on CSR and fixed-slot
// side records, N = 2 to 8, an empty matrix and a truncated image, and
// malformed fields and images.  Exit status 0 when every case round-trips and
// every malformed input is rejected with its status.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <random>
#include <vector>

#include "stagq.h"

// A finite normal fp16 bit pattern of magnitude between about 2^-10 and 2^-4
// (the weights' scale), random sign.
static uint16_t rand_half(std::mt19937& rng) {
  const uint32_t sign = rng() & 1u, expo = 5u + rng() % 7u, mant = rng() & 0x3ffu;
  return uint16_t((sign << 15) | (expo << 10) | mant);
}

static int run(int R, int C, int g, int N, double frac, int ppr, int slots, unsigned seed) {
  std::mt19937 rng(seed);
  const int64_t n = int64_t(R) * C;
  std::vector<uint16_t> w(size_t(n) + 1);
  for (int64_t i = 0; i < n; i++) w[size_t(i)] = rand_half(rng);
  const int64_t K = int64_t(frac * double(n) + 0.5);
  const int64_t cap = K + int64_t(R) * ppr + 1;
  std::vector<uint8_t> q(size_t(n) + 1), planes(size_t(N - 2) * size_t(n) + 1);
  std::vector<uint16_t> lo(size_t(n / g) + 1), s(size_t(n / g) + 1), val(static_cast<size_t>(cap));
  std::vector<int32_t> rp(size_t(R) + 1), col(static_cast<size_t>(cap));
  int64_t npre = 0;
  int st = stagq_encode(w.data(), R, C, g, N, K, 4.0, ppr, q.data(), planes.data(), lo.data(), s.data(),
                        rp.data(), col.data(), val.data(), &npre);
  if (st) { printf("encode: status %d\n", st); return 1; }
  const int64_t nnz = rp[size_t(R)];
  stagq_fields f{R, C, g, N, q.data(), planes.data(), lo.data(), s.data(), rp.data(), col.data(), val.data(),
                 nnz, nullptr, slots};
  const size_t bytes = stagq_packed_bytes(&f);
  if (!bytes) { printf("packed_bytes: 0\n"); return 1; }
  void* img = aligned_alloc(16, (bytes + 15) / 16 * 16);
  st = stagq_pack_host(&f, img, bytes);
  if (st) { printf("pack_host: status %d\n", st); free(img); return 1; }
  stagq_info info;
  std::vector<uint8_t> q2(q.size()), p2(planes.size());
  std::vector<uint16_t> lo2(lo.size()), s2(s.size()), v2(val.size());
  std::vector<int32_t> rp2(rp.size()), c2(col.size());
  st = stagq_unpack_host(img, bytes, &info, q2.data(), p2.data(), lo2.data(), s2.data(), rp2.data(), c2.data(),
                         v2.data());
  if (st) { printf("unpack_host: status %d\n", st); free(img); return 1; }
  bool ok = memcmp(q.data(), q2.data(), size_t(n)) == 0 &&
            memcmp(planes.data(), p2.data(), size_t(N - 2) * size_t(n)) == 0 &&
            memcmp(lo.data(), lo2.data(), size_t(n / g) * 2) == 0 && memcmp(s.data(), s2.data(), size_t(n / g) * 2) == 0 &&
            rp == rp2 && memcmp(col.data(), c2.data(), size_t(nnz) * 4) == 0 &&
            memcmp(val.data(), v2.data(), size_t(nnz) * 2) == 0;
  if (stagq_unpack_host(img, bytes - 1, &info, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == 0) {
    printf("a truncated image was accepted\n");
    ok = false;
  }
  printf("%d x %d g=%d N=%d nnz=%lld side_slots=%d: %s\n", R, C, g, N, (long long)nnz, info.side_slots,
         ok ? "round trip ok" : "MISMATCH");
  free(img);
  return ok ? 0 : 1;
}

// Malformed fields and images: each is rejected with its status, and nothing
// reads outside the arrays while finding that out.
static int malformed() {
  std::mt19937 rng(11);
  const int R = 20, C = 256, g = 64, N = 4;
  const int64_t n = int64_t(R) * C, K = 40;
  std::vector<uint16_t> w(static_cast<size_t>(n));
  for (auto& v : w) v = rand_half(rng);
  std::vector<uint8_t> q(static_cast<size_t>(n)), planes(static_cast<size_t>(2 * n));
  std::vector<uint16_t> lo(static_cast<size_t>(n / g)), s(static_cast<size_t>(n / g)), val(static_cast<size_t>(K));
  std::vector<int32_t> rp(static_cast<size_t>(R + 1)), col(static_cast<size_t>(K));
  int64_t npre = 0;
  if (stagq_encode(w.data(), R, C, g, N, K, 4.0, 0, q.data(), planes.data(), lo.data(), s.data(), rp.data(),
                   col.data(), val.data(), &npre))
    return 1;
  const stagq_fields good{R, C, g, N, q.data(), planes.data(), lo.data(), s.data(), rp.data(), col.data(),
                          val.data(), K, nullptr, 0};
  std::vector<uint8_t> buf(1 << 20);
  void* dst = buf.data() + (16 - reinterpret_cast<uintptr_t>(buf.data()) % 16) % 16;
  int fails = 0;
  auto expect = [&](const char* what, const stagq_fields& f, int want) {
    const int got = stagq_pack_host(&f, dst, 1 << 19);
    if (got != want) { printf("%s: status %d, expected %d\n", what, got, want); fails++; }
  };
  expect("good", good, STAGQ_OK);
  { auto r2 = rp; r2[R] = int32_t(K - 1); stagq_fields f = good; f.row_ptr = r2.data(); expect("row_ptr end", f, STAGQ_ECSR); }
  { auto r2 = rp; r2[5] = r2[4] - 1; stagq_fields f = good; f.row_ptr = r2.data(); expect("row_ptr order", f, STAGQ_ECSR); }
  { auto c2 = col; c2[0] = C; stagq_fields f = good; f.col = c2.data(); expect("column range", f, STAGQ_ECSR); }
  { auto q2 = q; q2[7] = 4; stagq_fields f = good; f.q = q2.data(); expect("base code", f, STAGQ_EFIELD); }
  {
    int r = 0;
    while (rp[size_t(r) + 1] == rp[size_t(r)]) r++;
    auto p2 = planes; p2[size_t(r) * C + size_t(col[size_t(rp[size_t(r)])])] = 1;
    stagq_fields f = good; f.planes = p2.data(); expect("plane at a held-out weight", f, STAGQ_EFIELD);
  }
  { auto l2 = lo; l2[3] = 0x7c00; stagq_fields f = good; f.lo = l2.data(); expect("infinite lo", f, STAGQ_EFIELD); }
  {
    int most = 0;
    for (int r = 0; r < R; r++) most = std::max(most, rp[size_t(r) + 1] - rp[size_t(r)]);
    stagq_fields f = good; f.side_slots = most - 1; expect("too few slots", f, STAGQ_ECSR);
  }
  // an image with a bad magic
  const size_t bytes = stagq_packed_bytes(&good);
  stagq_info info;
  {
    std::vector<uint8_t> im(bytes + 16);
    void* p = im.data() + (16 - reinterpret_cast<uintptr_t>(im.data()) % 16) % 16;
    if (stagq_pack_host(&good, p, bytes)) return 1;
    static_cast<uint8_t*>(p)[0] ^= 1;
    if (stagq_unpack_host(p, bytes, &info, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) !=
        STAGQ_EIMAGE) { printf("bad magic accepted\n"); fails++; }
  }
  printf("malformed inputs: %s\n", fails ? "FAILED" : "all rejected");
  return fails ? 1 : 0;
}

int main() {
  int bad = malformed();
  bad |= run(37, 384, 64, 4, 0.01, 0, 0, 1);
  bad |= run(37, 384, 64, 4, 0.01, 0, -1, 2);
  bad |= run(40, 512, 32, 6, 0.02, 3, -1, 3);
  bad |= run(16, 256, 128, 2, 0.0, 0, -1, 4);
  bad |= run(33, 1024, 128, 8, 0.005, 2, 7, 6);
  bad |= run(0, 256, 128, 4, 0.0, 0, 0, 7);
  return bad;
}
