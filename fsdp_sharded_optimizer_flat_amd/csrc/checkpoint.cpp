// checkpoint.cpp -- sharded checkpoints of the optimizer state, resharded
// when they are loaded.
//
// "ZeRO and FSDP sharding", Implementation notes: every rank writes its own
// shard of the checkpoint, and a checkpoint taken at one N is resharded to a
// different N at load time.  "Learn: ZeRO & FSDP", section 5: the same
// state carries over between the flat (FSDP1 / ZeRO) and the per-parameter
// dim-0 (FSDP2) layouts.
//
// One file per rank, little-endian:
//   FileHeader (64 bytes)            magic, versions, N, U, rank, step, sizes
//   U x (int64 numel, int64 granule) the layout's units
//   3 x S binary32                   master, exp_avg, exp_avg_sq (S = shard)
//   uint32 CRC-32C of all the bytes above, uint32 0
// The values are copied bit for bit.  A load rebuilds the saved layout from
// the unit table, checks every file against it, and fills the destination
// shard with the copy plan of the device reshard (build_reshard_runs): each
// run is one positioned read from the file of the rank that holds it, so a
// load reads only the bytes the destination needs and allocates no staging
// buffer.  CRC-32C: the Castagnoli polynomial (0x1EDC6F41, reflected
// 0x82F63B78), initial value and final xor 0xFFFFFFFF, computed with the
// SSE4.2 crc32 instruction.
#include <fcntl.h>
#include <nmmintrin.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "zero_internal.h"

namespace {

constexpr char kMagic[8] = {'Z', 'E', 'R', 'O', 'C', 'K', 'P', 'T'};
constexpr uint32_t kFormat = 1;
constexpr int32_t kArrays = 3;  // master, exp_avg, exp_avg_sq
constexpr int64_t kMaxShard = int64_t(1) << 56;  // keeps every file offset within int64

struct FileHeader {
    char magic[8];
    uint32_t format;
    uint32_t abi;
    int32_t n_ranks;
    int32_t n_units;
    int32_t rank;
    int32_t step;
    int64_t numel;   // sum of the units' numels
    int64_t shard;   // S: elements per array
    int32_t n_arrays;
    int32_t dtype;   // ZERO_F32
    int64_t reserved;
};
static_assert(sizeof(FileHeader) == 64, "fixed header size");

struct UnitRecord {
    int64_t numel, granule;
};

uint32_t crc32c_update(uint32_t crc, const void *data, size_t n)
{
    const unsigned char *p = static_cast<const unsigned char *>(data);
    uint64_t c = crc;
    while (n >= 8) {
        uint64_t w;
        std::memcpy(&w, p, 8);
        c = _mm_crc32_u64(c, w);
        p += 8;
        n -= 8;
    }
    uint32_t c32 = (uint32_t)c;
    while (n--)
        c32 = _mm_crc32_u8(c32, *p++);
    return c32;
}

// An open file descriptor closed on scope exit.
struct Fd {
    int fd = -1;
    explicit Fd(int f) : fd(f) {}
    ~Fd()
    {
        if (fd >= 0)
            ::close(fd);
    }
    Fd(const Fd &) = delete;
    Fd &operator=(const Fd &) = delete;
    Fd(Fd &&o) noexcept : fd(o.fd) { o.fd = -1; }
};

bool write_all(int fd, const void *buf, size_t n, uint32_t *crc)
{
    const char *p = static_cast<const char *>(buf);
    *crc = crc32c_update(*crc, buf, n);
    while (n > 0) {
        const ssize_t w = ::write(fd, p, n);
        if (w < 0 && errno == EINTR)
            continue;
        if (w <= 0)
            return false;
        p += w;
        n -= (size_t)w;
    }
    return true;
}

bool pread_all(int fd, void *buf, size_t n, int64_t off)
{
    char *p = static_cast<char *>(buf);
    while (n > 0) {
        const ssize_t r = ::pread(fd, p, n, (off_t)off);
        if (r < 0 && errno == EINTR)
            continue;
        if (r <= 0)
            return false;
        p += r;
        n -= (size_t)r;
        off += r;
    }
    return true;
}

int64_t payload_offset(int32_t n_units) { return (int64_t)sizeof(FileHeader) + 16 * (int64_t)n_units; }

int64_t file_bytes(int32_t n_units, int64_t shard)
{
    return payload_offset(n_units) + (int64_t)kArrays * shard * 4 + 8;
}

// One shard file's header and unit table, checked for internal consistency.
struct Saved {
    FileHeader h{};
    std::vector<UnitRecord> units;
};

zero_status read_header(int fd, Saved *s)
{
    if (!pread_all(fd, &s->h, sizeof s->h, 0))
        return ZERO_ECORRUPT;  // shorter than a header
    const FileHeader &h = s->h;
    if (std::memcmp(h.magic, kMagic, 8) != 0 || h.format != kFormat || h.n_arrays != kArrays ||
        h.dtype != ZERO_F32 || h.n_ranks < 1 || h.n_units < 0 || h.n_units > ZERO_MAX_UNITS ||
        h.rank < 0 || h.rank >= h.n_ranks || h.step < 0 || h.shard < 0 || h.numel < 0 ||
        h.shard > kMaxShard)
        return ZERO_ECORRUPT;
    s->units.resize((size_t)h.n_units);
    if (h.n_units > 0 && !pread_all(fd, s->units.data(), 16 * (size_t)h.n_units, sizeof h))
        return ZERO_ECORRUPT;
    struct stat st {};
    if (::fstat(fd, &st) != 0)
        return ZERO_EIO;
    if ((int64_t)st.st_size != file_bytes(h.n_units, h.shard))
        return ZERO_ECORRUPT;  // truncated or padded
    return ZERO_OK;
}

// The layout a header describes, rebuilt by the packer; ECORRUPT unless its
// totals are the header's.
zero_status saved_layout(const Saved &s, std::vector<char> &buf)
{
    std::vector<int64_t> numel(s.units.size()), gran(s.units.size());
    for (size_t u = 0; u < s.units.size(); ++u) {
        numel[u] = s.units[u].numel;
        gran[u] = s.units[u].granule;
    }
    buf.assign(zero_layout_bytes(s.h.n_units), 0);
    zero_layout *L = reinterpret_cast<zero_layout *>(buf.data());
    const zero_status st = zero_pack_rows(s.h.n_ranks, s.h.n_units, numel.data(), gran.data(), L,
                                          buf.size(), nullptr);
    if (st != ZERO_OK)
        return ZERO_ECORRUPT;
    if (L->numel != s.h.numel || L->shard != s.h.shard)
        return ZERO_ECORRUPT;
    return ZERO_OK;
}

zero_status verify_crc(int fd, int64_t size)
{
    // stream the file in 64 KiB pieces through a stack buffer
    char buf[1 << 16];
    uint32_t crc = 0xFFFFFFFFu;
    const int64_t body = size - 8;
    for (int64_t off = 0; off < body;) {
        const size_t n = (size_t)std::min<int64_t>(sizeof buf, body - off);
        if (!pread_all(fd, buf, n, off))
            return ZERO_EIO;
        crc = crc32c_update(crc, buf, n);
        off += (int64_t)n;
    }
    uint32_t trailer[2];
    if (!pread_all(fd, trailer, sizeof trailer, body))
        return ZERO_EIO;
    return (crc ^ 0xFFFFFFFFu) == trailer[0] && trailer[1] == 0 ? ZERO_OK : ZERO_ECORRUPT;
}

}  // namespace

extern "C" zero_status zero_ckpt_save(const char *path, const zero_layout *L, int32_t rank,
                                      int32_t step, const float *master, const float *exp_avg,
                                      const float *exp_avg_sq)
{
    if (!path || !zero::layout_ok(L) || rank < 0 || rank >= L->n_ranks || step < 0)
        return ZERO_EINVAL;
    const int64_t S = L->shard;
    if (S > 0 && (!master || !exp_avg || !exp_avg_sq))
        return ZERO_EINVAL;
    FileHeader h{};
    std::memcpy(h.magic, kMagic, 8);
    h.format = kFormat;
    h.abi = ZERO_ABI_VERSION;
    h.n_ranks = L->n_ranks;
    h.n_units = L->n_units;
    h.rank = rank;
    h.step = step;
    h.numel = L->numel;
    h.shard = S;
    h.n_arrays = kArrays;
    h.dtype = ZERO_F32;
    std::vector<UnitRecord> units((size_t)L->n_units);
    for (int32_t u = 0; u < L->n_units; ++u)
        units[(size_t)u] = {L->unit[u].numel, L->unit[u].granule};

    // written to a temporary name, then renamed: a reader never sees half a file
    const std::string tmp = std::string(path) + ".tmp";
    {
        Fd f(::open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644));
        if (f.fd < 0)
            return ZERO_EIO;
        uint32_t crc = 0xFFFFFFFFu;
        bool ok = write_all(f.fd, &h, sizeof h, &crc) &&
                  (units.empty() || write_all(f.fd, units.data(), 16 * units.size(), &crc));
        const float *arrays[kArrays] = {master, exp_avg, exp_avg_sq};
        for (int a = 0; ok && a < kArrays; ++a)
            ok = S == 0 || write_all(f.fd, arrays[a], (size_t)S * 4, &crc);
        const uint32_t trailer[2] = {crc ^ 0xFFFFFFFFu, 0u};
        uint32_t unused = 0;
        ok = ok && write_all(f.fd, trailer, sizeof trailer, &unused) && ::fdatasync(f.fd) == 0;
        if (!ok) {
            ::unlink(tmp.c_str());
            return ZERO_EIO;
        }
    }
    if (::rename(tmp.c_str(), path) != 0) {
        ::unlink(tmp.c_str());
        return ZERO_EIO;
    }
    return ZERO_OK;
}

extern "C" zero_status zero_ckpt_inspect(const char *path, int32_t verify, zero_ckpt_info *info,
                                         zero_layout *layout, size_t layout_bytes,
                                         size_t *bytes_needed)
{
    if (!path || !info)
        return ZERO_EINVAL;
    Fd f(::open(path, O_RDONLY | O_CLOEXEC));
    if (f.fd < 0)
        return ZERO_EIO;
    Saved s;
    zero_status st = read_header(f.fd, &s);
    if (st != ZERO_OK)
        return st;
    std::vector<char> lb;
    if ((st = saved_layout(s, lb)) != ZERO_OK)
        return st;
    if (verify && (st = verify_crc(f.fd, file_bytes(s.h.n_units, s.h.shard))) != ZERO_OK)
        return st;
    zero_ckpt_info o{};
    o.format = (int32_t)s.h.format;
    o.abi = (int32_t)s.h.abi;
    o.n_ranks = s.h.n_ranks;
    o.n_units = s.h.n_units;
    o.rank = s.h.rank;
    o.step = s.h.step;
    o.numel = s.h.numel;
    o.shard = s.h.shard;
    *info = o;
    if (bytes_needed)
        *bytes_needed = lb.size();
    if (layout) {
        if (layout_bytes < lb.size())
            return ZERO_ENOSPC;
        std::memcpy(layout, lb.data(), lb.size());
    }
    return ZERO_OK;
}

extern "C" zero_status zero_ckpt_load(const char *const *paths, int32_t n_files,
                                      const zero_layout *to, int32_t dst_rank, int32_t verify,
                                      int32_t *step, float *master, float *exp_avg,
                                      float *exp_avg_sq)
{
    if (!paths || n_files < 1 || n_files > ZERO_MAX_UNITS || !zero::layout_ok(to) ||
        dst_rank < 0 || dst_rank >= to->n_ranks)
        return ZERO_EINVAL;
    if (to->shard > 0 && (!master || !exp_avg || !exp_avg_sq))
        return ZERO_EINVAL;
    for (int32_t q = 0; q < n_files; ++q)
        if (!paths[q])
            return ZERO_EINVAL;
    // every file: one checkpoint's rank q, all with the same layout and step
    std::vector<Fd> fds;
    fds.reserve((size_t)n_files);
    Saved first;
    for (int32_t q = 0; q < n_files; ++q) {
        fds.emplace_back(::open(paths[q], O_RDONLY | O_CLOEXEC));
        if (fds.back().fd < 0)
            return ZERO_EIO;
        Saved s;
        zero_status st = read_header(fds.back().fd, &s);
        if (st != ZERO_OK)
            return st;
        if (q == 0) {
            if (s.h.n_ranks != n_files)
                return ZERO_EINVAL;  // the checkpoint has another number of shards
            first = s;
        } else if (s.h.n_ranks != first.h.n_ranks || s.h.n_units != first.h.n_units ||
                   s.h.step != first.h.step || s.h.shard != first.h.shard ||
                   std::memcmp(s.units.data(), first.units.data(), 16 * s.units.size()) != 0) {
            return ZERO_ECORRUPT;  // files of different checkpoints
        }
        if (s.h.rank != q)
            return ZERO_EINVAL;  // paths[q] must be rank q's shard
        if (verify && (st = verify_crc(fds.back().fd, file_bytes(s.h.n_units, s.h.shard))) !=
                          ZERO_OK)
            return st;
    }
    std::vector<char> lb;
    zero_status st = saved_layout(first, lb);
    if (st != ZERO_OK)
        return st;
    const zero_layout *from = reinterpret_cast<const zero_layout *>(lb.data());
    if (!zero::layouts_match(from, to))
        return ZERO_EINVAL;  // the destination holds another number of elements

    const std::vector<zero::ReshardRun> runs = zero::build_reshard_runs(from, to, dst_rank);
    const int64_t S_from = from->shard, base = payload_offset(from->n_units);
    float *dst[kArrays] = {master, exp_avg, exp_avg_sq};
    for (int a = 0; a < kArrays; ++a) {
        for (const zero::ReshardRun &r : runs) {
            float *d = dst[a] + r.dst_k;
            if (r.src_rank < 0) {
                std::memset(d, 0, (size_t)r.len * 4);  // padding
                continue;
            }
            const int64_t off = base + ((int64_t)a * S_from + r.src_k) * 4;
            if (!pread_all(fds[(size_t)r.src_rank].fd, d, (size_t)r.len * 4, off))
                return ZERO_EIO;
        }
    }
    if (step)
        *step = first.h.step;
    return ZERO_OK;
}
