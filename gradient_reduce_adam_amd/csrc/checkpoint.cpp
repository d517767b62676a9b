// Checkpoint and resume of the step's state with resharding (dpckpt.h): the
// shard file format, the manifest and its atomic commit, and the staging
// between a plan's device memory and the files.
#include <dirent.h>
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cinttypes>
#include <cstdio>
#include <cstring>
#include <functional>
#include <memory>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "dpckpt.h"
#include "plan.h"

using dpapi::fail;
using dpapi::hip_fail;

namespace {

constexpr char kMagic[8] = {'D', 'P', 'S', 'H', 'A', 'R', 'D', '1'};
constexpr uint32_t kVersion = 1;
constexpr int64_t kBlockElems = int64_t{1} << 20;  // elements per checksum block
constexpr int64_t kStageElems = 16 * kBlockElems;  // elements per staged piece (64 MiB of binary32)
constexpr uint64_t kAlign = 4096;                  // arrays start on this boundary
constexpr int kArrays = 4;                         // master, exp_avg, exp_avg_sq, param
const char* const kManifest = "manifest.dpck";

// ---- checksums --------------------------------------------------------------
// Corruption check, not a cryptographic hash: four interleaved lanes of
// multiply-xorshift over 8-byte words, then the lanes and the length mixed by
// the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014).
uint64_t fmix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t checksum(const void* data, size_t n) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    const uint64_t k = 0x9E3779B97F4A7C15ull;
    uint64_t h[4] = {1, 2, 3, 4};
    const size_t words = n / 8;
    size_t i = 0;
    for (; i + 4 <= words; i += 4) {
        for (int j = 0; j < 4; ++j) {
            uint64_t w;
            std::memcpy(&w, p + 8 * (i + j), 8);
            h[j] = (h[j] ^ w) * k;
            h[j] ^= h[j] >> 29;
        }
    }
    for (; i < words; ++i) {
        uint64_t w;
        std::memcpy(&w, p + 8 * i, 8);
        h[i & 3] = (h[i & 3] ^ w) * k;
        h[i & 3] ^= h[i & 3] >> 29;
    }
    uint64_t tail = 0;
    std::memcpy(&tail, p + 8 * words, n % 8);
    return fmix(fmix(h[0] ^ tail) ^ fmix(h[1] + 1) ^ fmix(h[2] + 2) ^ fmix(h[3] + 3) ^ n);
}

uint64_t layout_hash(const dp_layout* L) {
    std::vector<int64_t> v(L->numel, L->numel + L->num_tensors);
    v.push_back(L->num_tensors);
    return checksum(v.data(), v.size() * sizeof(int64_t));
}

size_t esize(int array, dp_dtype pdt) { return array < 3 ? 4 : (pdt == DP_F32 ? 4 : 2); }

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---- the shard file -----------------------------------------------------------
struct ShardHeader {
    char magic[8];
    uint32_t version;
    int32_t param_dtype;
    int64_t generation, params, begin, end;
    uint64_t layout_hash;
    int64_t block_elems, nblocks;  // checksum blocks per array
    uint64_t offsets[kArrays];     // byte offset of each array
    uint64_t file_bytes;
    uint64_t check;                // checksum of the bytes above
    char pad[256 - 120];
};
static_assert(sizeof(ShardHeader) == 256, "the shard header is 256 bytes");

uint64_t header_check(const ShardHeader& h) { return checksum(&h, offsetof(ShardHeader, check)); }

ShardHeader make_header(int64_t gen, const dp_layout* L, int64_t P, int64_t begin, int64_t end) {
    ShardHeader h;
    std::memset(&h, 0, sizeof(h));
    std::memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.param_dtype = L->param_dtype;
    h.generation = gen;
    h.params = P;
    h.begin = begin;
    h.end = end;
    h.layout_hash = layout_hash(L);
    h.block_elems = kBlockElems;
    const int64_t count = end - begin;
    h.nblocks = (count + kBlockElems - 1) / kBlockElems;
    uint64_t off = align_up(sizeof(ShardHeader) + static_cast<uint64_t>(kArrays * h.nblocks) * 8);
    for (int a = 0; a < kArrays; ++a) {
        h.offsets[a] = off;
        off = align_up(off + static_cast<uint64_t>(count) * esize(a, L->param_dtype));
    }
    h.file_bytes = off;
    h.check = header_check(h);
    return h;
}

std::string shard_name(int64_t gen, int64_t begin, int64_t end) {
    char buf[96];
    std::snprintf(buf, sizeof(buf), "g%" PRId64 "-%" PRId64 "-%" PRId64 ".dpshard", gen, begin, end);
    return buf;
}

// parses "g<gen>-<begin>-<end>.dpshard"
bool parse_shard_name(const char* name, int64_t* gen, int64_t* begin, int64_t* end) {
    long long g, b, e;
    int used = 0;
    if (std::sscanf(name, "g%lld-%lld-%lld.dpshard%n", &g, &b, &e, &used) != 3) return false;
    if (name[used] != '\0') return false;
    *gen = g;
    *begin = b;
    *end = e;
    return shard_name(g, b, e) == name;
}

std::string join(const std::string& dir, const std::string& name) { return dir + "/" + name; }

// ---- small POSIX helpers --------------------------------------------------------
struct Fd {
    int fd = -1;
    explicit Fd(int f) : fd(f) {}
    ~Fd() {
        if (fd >= 0) ::close(fd);
    }
    Fd(const Fd&) = delete;
    Fd& operator=(const Fd&) = delete;
};

// Removes a writer's temporary file unless it was renamed into place.
struct TmpFile {
    std::string path;
    bool renamed = false;
    explicit TmpFile(std::string p) : path(std::move(p)) {}
    ~TmpFile() {
        if (!renamed) (void)::unlink(path.c_str());
    }
    TmpFile(const TmpFile&) = delete;
    TmpFile& operator=(const TmpFile&) = delete;
};

dp_status io_fail(const char* what, const std::string& path) {
    return fail(DP_ERR_IO, "%s %s: %s", what, path.c_str(), std::strerror(errno));
}

dp_status write_all(int fd, const void* buf, size_t n, uint64_t off, const std::string& path) {
    const char* p = static_cast<const char*>(buf);
    while (n > 0) {
        const ssize_t w = ::pwrite(fd, p, n, static_cast<off_t>(off));
        if (w < 0) {
            if (errno == EINTR) continue;
            return io_fail("write", path);
        }
        p += w;
        n -= static_cast<size_t>(w);
        off += static_cast<uint64_t>(w);
    }
    return DP_OK;
}

dp_status read_all(int fd, void* buf, size_t n, uint64_t off, const std::string& path) {
    char* p = static_cast<char*>(buf);
    while (n > 0) {
        const ssize_t r = ::pread(fd, p, n, static_cast<off_t>(off));
        if (r < 0) {
            if (errno == EINTR) continue;
            return io_fail("read", path);
        }
        if (r == 0) return fail(DP_ERR_CORRUPT, "%s is shorter than its header says", path.c_str());
        p += r;
        n -= static_cast<size_t>(r);
        off += static_cast<uint64_t>(r);
    }
    return DP_OK;
}

dp_status sync_dir(const std::string& dir) {
    Fd d(::open(dir.c_str(), O_RDONLY | O_DIRECTORY));
    if (d.fd < 0) return io_fail("open directory", dir);
    if (::fsync(d.fd) != 0) return io_fail("fsync directory", dir);
    return DP_OK;
}

// Writes `data` to dir/name through a temporary file, flushed and renamed.
dp_status replace_file(const std::string& dir, const std::string& name, const std::string& data) {
    TmpFile tf(join(dir, ".tmp-" + name + "." + std::to_string(::getpid())));
    const std::string& tmp = tf.path;
    const std::string dst = join(dir, name);
    {
        Fd f(::open(tmp.c_str(), O_CREAT | O_TRUNC | O_WRONLY, 0644));
        if (f.fd < 0) return io_fail("create", tmp);
        dp_status s = write_all(f.fd, data.data(), data.size(), 0, tmp);
        if (s != DP_OK) return s;
        if (::fsync(f.fd) != 0) return io_fail("fsync", tmp);
    }
    if (::rename(tmp.c_str(), dst.c_str()) != 0) return io_fail("rename to", dst);
    tf.renamed = true;
    return sync_dir(dir);
}

dp_status read_text(const std::string& path, std::string* out) {
    Fd f(::open(path.c_str(), O_RDONLY));
    if (f.fd < 0) {
        if (errno == ENOENT) return fail(DP_ERR_STATE, "no committed checkpoint: %s does not exist", path.c_str());
        return io_fail("open", path);
    }
    struct stat st;
    if (::fstat(f.fd, &st) != 0) return io_fail("stat", path);
    out->resize(static_cast<size_t>(st.st_size));
    return read_all(f.fd, &(*out)[0], out->size(), 0, path);
}

// ---- the manifest ----------------------------------------------------------------
struct ShardRef {
    int64_t begin, end;
    std::string name;
    uint64_t file_bytes, check;
};

struct Manifest {
    int64_t generation = 0, params = 0;
    int32_t param_dtype = 0;
    std::vector<int64_t> numel;
    uint64_t layout_hash = 0;
    dp_step_state state{};
    dp_state_cfg cfg{};
    std::vector<ShardRef> shards;
};

uint64_t bits(double x) {
    uint64_t u;
    std::memcpy(&u, &x, 8);
    return u;
}

double from_bits(uint64_t u) {
    double x;
    std::memcpy(&x, &u, 8);
    return x;
}

std::string format_manifest(const Manifest& m) {
    std::string s;
    char buf[512];
    auto add = [&](const char* fmt, auto... args) {
        std::snprintf(buf, sizeof(buf), fmt, args...);
        s += buf;
    };
    add("dpckpt %u\n", kVersion);
    add("generation %" PRId64 "\n", m.generation);
    add("params %" PRId64 "\n", m.params);
    add("param_dtype %d\n", m.param_dtype);
    add("tensors %zu\n", m.numel.size());
    s += "numel";
    for (int64_t x : m.numel) add(" %" PRId64, x);
    s += "\n";
    add("layout_hash %016" PRIx64 "\n", m.layout_hash);
    const dp_step_state& t = m.state;
    add("state %" PRId64 " %" PRId64 " %" PRId64 " %d %016" PRIx64 " %016" PRIx64 " %016" PRIx64 " %016" PRIx64
        " %016" PRIx64 " %016" PRIx64 " %016" PRIx64 "\n",
        t.t, t.iter, t.growth_tracker, t.found_inf, bits(t.beta1_pow), bits(t.beta2_pow), bits(t.scale),
        bits(t.sumsq), bits(t.norm), bits(t.clip), bits(t.gscale));
    const dp_state_cfg& c = m.cfg;
    add("cfg %016" PRIx64 " %016" PRIx64 " %d %d %016" PRIx64 " %016" PRIx64 " %016" PRIx64 "\n", bits(c.beta1),
        bits(c.beta2), c.scaler_mode, c.growth_interval, bits(c.init_scale), bits(c.backoff), bits(c.growth));
    add("shards %zu\n", m.shards.size());
    for (const ShardRef& r : m.shards)
        add("shard %" PRId64 " %" PRId64 " %s %" PRIu64 " %016" PRIx64 "\n", r.begin, r.end, r.name.c_str(),
            r.file_bytes, r.check);
    add("check %016" PRIx64 "\n", checksum(s.data(), s.size()));
    return s;
}

dp_status parse_manifest(const std::string& path, const std::string& text, Manifest* m) {
    const size_t at = text.rfind("check ");
    if (at == std::string::npos || (at > 0 && text[at - 1] != '\n'))
        return fail(DP_ERR_CORRUPT, "%s has no checksum line", path.c_str());
    unsigned long long want = 0;
    if (std::sscanf(text.c_str() + at, "check %16llx", &want) != 1 || checksum(text.data(), at) != want)
        return fail(DP_ERR_CORRUPT, "%s fails its checksum", path.c_str());
    const char* p = text.c_str();
    auto line_end = [&]() {
        const char* e = std::strchr(p, '\n');
        return e ? e : p + std::strlen(p);
    };
    auto next_line = [&]() {
        const char* e = line_end();
        p = *e ? e + 1 : e;
    };
    auto bad = [&](const char* what) { return fail(DP_ERR_CORRUPT, "%s: bad %s line", path.c_str(), what); };
    unsigned ver = 0;
    if (std::sscanf(p, "dpckpt %u", &ver) != 1 || ver != kVersion) return bad("version");
    next_line();
    long long g, P;
    int pdt;
    size_t T;
    if (std::sscanf(p, "generation %lld", &g) != 1) return bad("generation");
    next_line();
    if (std::sscanf(p, "params %lld", &P) != 1) return bad("params");
    next_line();
    if (std::sscanf(p, "param_dtype %d", &pdt) != 1) return bad("param_dtype");
    next_line();
    if (std::sscanf(p, "tensors %zu", &T) != 1) return bad("tensors");
    next_line();
    m->generation = g;
    m->params = P;
    m->param_dtype = pdt;
    if (std::strncmp(p, "numel", 5) != 0) return bad("numel");
    {
        const char* e = line_end();
        const char* q = p + 5;
        m->numel.clear();
        while (q < e) {
            char* stop = nullptr;
            const long long x = std::strtoll(q, &stop, 10);
            if (stop == q) break;
            m->numel.push_back(x);
            q = stop;
        }
        if (m->numel.size() != T) return bad("numel");
    }
    next_line();
    unsigned long long lh;
    if (std::sscanf(p, "layout_hash %16llx", &lh) != 1) return bad("layout_hash");
    m->layout_hash = lh;
    next_line();
    {
        long long t, it, gt;
        int fi;
        unsigned long long b1, b2, sc, ss, nm, cl, gs;
        if (std::sscanf(p, "state %lld %lld %lld %d %16llx %16llx %16llx %16llx %16llx %16llx %16llx", &t, &it, &gt,
                        &fi, &b1, &b2, &sc, &ss, &nm, &cl, &gs) != 11)
            return bad("state");
        dp_step_state& s = m->state;
        std::memset(&s, 0, sizeof(s));
        s.t = t;
        s.iter = it;
        s.growth_tracker = gt;
        s.found_inf = fi;
        s.beta1_pow = from_bits(b1);
        s.beta2_pow = from_bits(b2);
        s.scale = from_bits(sc);
        s.sumsq = from_bits(ss);
        s.norm = from_bits(nm);
        s.clip = from_bits(cl);
        s.gscale = from_bits(gs);
    }
    next_line();
    {
        unsigned long long b1, b2, is, bo, gr;
        int mode, gi;
        if (std::sscanf(p, "cfg %16llx %16llx %d %d %16llx %16llx %16llx", &b1, &b2, &mode, &gi, &is, &bo, &gr) != 7)
            return bad("cfg");
        dp_state_cfg& c = m->cfg;
        std::memset(&c, 0, sizeof(c));
        c.beta1 = from_bits(b1);
        c.beta2 = from_bits(b2);
        c.scaler_mode = mode;
        c.growth_interval = gi;
        c.init_scale = from_bits(is);
        c.backoff = from_bits(bo);
        c.growth = from_bits(gr);
    }
    next_line();
    size_t ns = 0;
    if (std::sscanf(p, "shards %zu", &ns) != 1) return bad("shards");
    next_line();
    m->shards.clear();
    for (size_t i = 0; i < ns; ++i) {
        long long b, e;
        char name[128];
        unsigned long long fb, ck;
        if (std::sscanf(p, "shard %lld %lld %127s %llu %16llx", &b, &e, name, &fb, &ck) != 5) return bad("shard");
        m->shards.push_back(ShardRef{b, e, name, fb, ck});
        next_line();
    }
    return DP_OK;
}

dp_status check_layout(const dp_layout* L, const char* where) {
    if (!L) return fail(DP_ERR_INVALID_ARG, "%s: null layout", where);
    if (L->num_tensors < 0 || (L->num_tensors > 0 && !L->numel))
        return fail(DP_ERR_BAD_LAYOUT, "%s: bad tensor list", where);
    if (L->param_dtype != DP_F16 && L->param_dtype != DP_BF16)
        return fail(DP_ERR_BAD_LAYOUT, "%s: param_dtype must be DP_F16 or DP_BF16", where);
    for (int32_t i = 0; i < L->num_tensors; ++i)
        if (L->numel[i] < 0) return fail(DP_ERR_BAD_LAYOUT, "%s: numel[%d] < 0", where, i);
    return DP_OK;
}

int64_t layout_params(const dp_layout* L) {
    int64_t P = 0;
    for (int32_t i = 0; i < L->num_tensors; ++i) P += L->numel[i];
    return P;
}

// Opens a shard file and checks its header against what the caller expects.
dp_status open_shard(const std::string& path, int64_t gen, const dp_layout* L, int64_t P, int64_t begin, int64_t end,
                     int* fd_out, ShardHeader* h) {
    const int fd = ::open(path.c_str(), O_RDONLY);
    if (fd < 0) return io_fail("open", path);
    Fd f(fd);
    dp_status s = read_all(fd, h, sizeof(*h), 0, path);
    if (s != DP_OK) return s;
    if (std::memcmp(h->magic, kMagic, 8) != 0 || h->version != kVersion || h->check != header_check(*h))
        return fail(DP_ERR_CORRUPT, "%s: bad shard header", path.c_str());
    if (h->generation != gen || h->params != P || h->begin != begin || h->end != end ||
        h->layout_hash != layout_hash(L) || h->param_dtype != L->param_dtype || h->block_elems != kBlockElems)
        return fail(DP_ERR_CORRUPT, "%s: header does not match the checkpoint", path.c_str());
    struct stat st;
    if (::fstat(fd, &st) != 0) return io_fail("stat", path);
    if (static_cast<uint64_t>(st.st_size) != h->file_bytes)
        return fail(DP_ERR_CORRUPT, "%s: %lld bytes, header says %llu", path.c_str(), static_cast<long long>(st.st_size),
                    static_cast<unsigned long long>(h->file_bytes));
    f.fd = -1;  // ownership to the caller
    *fd_out = fd;
    return DP_OK;
}

// Where shard data comes from and goes to.  get(array, lo, hi, staging, &ptr)
// makes elements [lo, hi) of an array available at *ptr (inside staging, or
// elsewhere); put(array, lo, hi, src) stores them.
using GetFn = std::function<dp_status(int, int64_t, int64_t, void*, const void**)>;
using PutFn = std::function<dp_status(int, int64_t, int64_t, const void*)>;

dp_status write_shard(const std::string& dir, int64_t gen, const dp_layout* L, int64_t begin, int64_t end,
                      void* staging, const GetFn& get) {
    const int64_t P = layout_params(L);
    if (begin < 0 || end > P || begin > end)
        return fail(DP_ERR_RANGE, "shard [%lld, %lld) not inside [0, %lld)", static_cast<long long>(begin),
                    static_cast<long long>(end), static_cast<long long>(P));
    if (gen < 0) return fail(DP_ERR_INVALID_ARG, "generation %lld < 0", static_cast<long long>(gen));
    const ShardHeader h = make_header(gen, L, P, begin, end);
    const std::string name = shard_name(gen, begin, end);
    TmpFile tf(join(dir, ".tmp-" + name + "." + std::to_string(::getpid())));
    const std::string& tmp = tf.path;
    Fd f(::open(tmp.c_str(), O_CREAT | O_TRUNC | O_WRONLY, 0644));
    if (f.fd < 0) return io_fail("create", tmp);
    std::vector<uint64_t> sums(static_cast<size_t>(kArrays * h.nblocks));
    for (int a = 0; a < kArrays; ++a) {
        const size_t es = esize(a, static_cast<dp_dtype>(L->param_dtype));
        for (int64_t lo = begin; lo < end; lo += kStageElems) {
            const int64_t hi = std::min(end, lo + kStageElems);
            const void* src = nullptr;
            dp_status s = get(a, lo, hi, staging, &src);
            if (s != DP_OK) return s;
            for (int64_t b = lo; b < hi; b += kBlockElems) {
                const int64_t bh = std::min(hi, b + kBlockElems);
                sums[static_cast<size_t>(a * h.nblocks + (b - begin) / kBlockElems)] =
                    checksum(static_cast<const char*>(src) + (b - lo) * es, static_cast<size_t>(bh - b) * es);
            }
            s = write_all(f.fd, src, static_cast<size_t>(hi - lo) * es,
                          h.offsets[a] + static_cast<uint64_t>(lo - begin) * es, tmp);
            if (s != DP_OK) return s;
        }
    }
    dp_status s = write_all(f.fd, &h, sizeof(h), 0, tmp);
    if (s == DP_OK && !sums.empty()) s = write_all(f.fd, sums.data(), sums.size() * 8, sizeof(h), tmp);
    if (s != DP_OK) return s;
    if (::ftruncate(f.fd, static_cast<off_t>(h.file_bytes)) != 0) return io_fail("truncate", tmp);
    if (::fsync(f.fd) != 0) return io_fail("fsync", tmp);
    if (::rename(tmp.c_str(), join(dir, name).c_str()) != 0) return io_fail("rename", tmp);
    tf.renamed = true;
    return DP_OK;
}

dp_status commit(const std::string& dir, int64_t gen, const dp_layout* L, const dp_step_state* scalars,
                 const dp_state_cfg* cfg) {
    const int64_t P = layout_params(L);
    std::vector<ShardRef> found;
    std::vector<std::string> stale;  // shard files of older generations
    {
        DIR* d = ::opendir(dir.c_str());
        if (!d) return io_fail("open directory", dir);
        while (dirent* e = ::readdir(d)) {
            int64_t g, b, en;
            const std::string name = e->d_name;
            if (parse_shard_name(name.c_str(), &g, &b, &en)) {
                if (g == gen) found.push_back(ShardRef{b, en, name, 0, 0});
                else if (g < gen) stale.push_back(name);
            } else if (name.compare(0, 5, ".tmp-") == 0) {
                // a writer's temporary file ".tmp-<shard name>.<pid>": left by a
                // writer that stopped, once its generation is older than this one
                const size_t dot = name.rfind('.');
                if (dot > 5 && parse_shard_name(name.substr(5, dot - 5).c_str(), &g, &b, &en) && g < gen)
                    stale.push_back(name);
            }
        }
        ::closedir(d);
    }
    std::sort(found.begin(), found.end(),
              [](const ShardRef& x, const ShardRef& y) { return x.begin != y.begin ? x.begin < y.begin : x.end < y.end; });
    int64_t cur = 0;
    for (ShardRef& r : found) {
        if (r.begin < 0 || r.end > P || r.begin > r.end)
            return fail(DP_ERR_STATE, "shard %s lies outside [0, %lld)", r.name.c_str(), static_cast<long long>(P));
        if (r.begin == r.end) continue;
        if (r.begin != cur)
            return fail(DP_ERR_STATE, "generation %lld: shards %s at %lld (gap or overlap)",
                        static_cast<long long>(gen), r.begin > cur ? "leave a gap" : "overlap",
                        static_cast<long long>(std::min(cur, r.begin)));
        cur = r.end;
    }
    if (cur != P)
        return fail(DP_ERR_STATE, "generation %lld: shards cover [0, %lld) of [0, %lld)", static_cast<long long>(gen),
                    static_cast<long long>(cur), static_cast<long long>(P));
    Manifest m;
    m.generation = gen;
    m.params = P;
    m.param_dtype = L->param_dtype;
    m.numel.assign(L->numel, L->numel + L->num_tensors);
    m.layout_hash = layout_hash(L);
    m.state = *scalars;
    m.cfg = *cfg;
    for (ShardRef& r : found) {
        int fd = -1;
        ShardHeader h;
        dp_status s = open_shard(join(dir, r.name), gen, L, P, r.begin, r.end, &fd, &h);
        if (s != DP_OK) return s;
        ::close(fd);
        r.file_bytes = h.file_bytes;
        r.check = h.check;
        m.shards.push_back(r);
    }
    dp_status s = replace_file(dir, kManifest, format_manifest(m));
    if (s != DP_OK) return s;
    for (const std::string& n : stale) (void)::unlink(join(dir, n).c_str());
    return DP_OK;
}

dp_status read_range(const std::string& dir, const dp_layout* L, int64_t begin, int64_t end, void* staging,
                     const PutFn& put, bool want[kArrays], dp_step_state* scalars, dp_state_cfg* cfg,
                     int64_t* generation) {
    const std::string mpath = join(dir, kManifest);
    std::string text;
    dp_status s = read_text(mpath, &text);
    if (s != DP_OK) return s;
    Manifest m;
    s = parse_manifest(mpath, text, &m);
    if (s != DP_OK) return s;
    const int64_t P = layout_params(L);
    if (m.params != P || m.param_dtype != L->param_dtype ||
        m.numel != std::vector<int64_t>(L->numel, L->numel + L->num_tensors) || m.layout_hash != layout_hash(L))
        return fail(DP_ERR_BAD_LAYOUT, "the checkpoint in %s was written for another tensor list or param dtype",
                    dir.c_str());
    if (begin < 0 || end > P || begin > end)
        return fail(DP_ERR_RANGE, "range [%lld, %lld) not inside [0, %lld)", static_cast<long long>(begin),
                    static_cast<long long>(end), static_cast<long long>(P));
    for (const ShardRef& r : m.shards) {
        const int64_t lo = std::max(begin, r.begin), hi = std::min(end, r.end);
        if (lo >= hi) continue;
        int fd = -1;
        ShardHeader h;
        const std::string path = join(dir, r.name);
        s = open_shard(path, m.generation, L, P, r.begin, r.end, &fd, &h);
        if (s != DP_OK) return s;
        Fd f(fd);
        if (h.check != r.check) return fail(DP_ERR_CORRUPT, "%s differs from the manifest's record", path.c_str());
        std::vector<uint64_t> sums(static_cast<size_t>(kArrays * h.nblocks));
        if (!sums.empty()) {
            s = read_all(fd, sums.data(), sums.size() * 8, sizeof(h), path);
            if (s != DP_OK) return s;
        }
        for (int a = 0; a < kArrays; ++a) {
            if (!want[a]) continue;
            const size_t es = esize(a, static_cast<dp_dtype>(L->param_dtype));
            // the whole checksum blocks around [lo, hi), a staged piece at a time
            const int64_t b0 = (lo - r.begin) / kBlockElems * kBlockElems + r.begin;
            const int64_t b1 = std::min(r.end, (hi - r.begin + kBlockElems - 1) / kBlockElems * kBlockElems + r.begin);
            for (int64_t x = b0; x < b1; x += kStageElems) {
                const int64_t xe = std::min(b1, x + kStageElems);
                s = read_all(fd, staging, static_cast<size_t>(xe - x) * es,
                             h.offsets[a] + static_cast<uint64_t>(x - r.begin) * es, path);
                if (s != DP_OK) return s;
                for (int64_t b = x; b < xe; b += kBlockElems) {
                    const int64_t bh = std::min(xe, b + kBlockElems);
                    const uint64_t got = checksum(static_cast<const char*>(staging) + (b - x) * es,
                                                 static_cast<size_t>(bh - b) * es);
                    if (got != sums[static_cast<size_t>(a * h.nblocks + (b - r.begin) / kBlockElems)])
                        return fail(DP_ERR_CORRUPT, "%s: array %d, elements [%lld, %lld) fail their checksum",
                                    path.c_str(), a, static_cast<long long>(b), static_cast<long long>(bh));
                }
                const int64_t ulo = std::max(lo, x), uhi = std::min(hi, xe);
                if (ulo < uhi) {
                    s = put(a, ulo, uhi, static_cast<const char*>(staging) + (ulo - x) * es);
                    if (s != DP_OK) return s;
                }
            }
        }
    }
    if (scalars) *scalars = m.state;
    if (cfg) *cfg = m.cfg;
    if (generation) *generation = m.generation;
    return DP_OK;
}

// ---- device staging ---------------------------------------------------------------
struct Pinned {
    void* p = nullptr;
    ~Pinned() {
        if (p) (void)hipHostFree(p);
    }
};

// Staging sizes, in bytes (binary32 elements; the widest array).  A save of
// [begin, end) stages at most kStageElems elements at a time; a read of
// [begin, end) stages the whole checksum blocks around each shard's part of
// it, which reach at most one block past either end.
size_t save_staging_bytes(int64_t begin, int64_t end) {
    const int64_t n = begin >= 0 && end > begin ? end - begin : 1;  // a bad range fails later
    return static_cast<size_t>(std::min(kStageElems, n)) * 4;
}

size_t read_staging_bytes(int64_t begin, int64_t end) {
    const int64_t n = begin >= 0 && end > begin ? end - begin : 0;  // a bad range fails later
    return static_cast<size_t>(std::min(kStageElems, n + 2 * kBlockElems)) * 4;
}

dp_status alloc_pinned(Pinned* b, size_t bytes) {
    hipError_t e = hipHostMalloc(&b->p, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        b->p = nullptr;
        return fail(DP_ERR_OOM, "hipHostMalloc of a %zu-byte staging buffer: %s", bytes, hipGetErrorString(e));
    }
    return DP_OK;
}

// Copies elements [lo, hi) of a role between its memory and a host buffer,
// one copy per contiguous segment (one for a flat binding, one per tensor
// piece for per-tensor bindings).  to_host selects the direction.  The role's
// memory may be device memory or pinned host memory (an offloaded state): the
// runtime tells them apart by address.
dp_status copy_role(const dp_plan* p, const dpapi::Binding& b, size_t es, int64_t lo, int64_t hi, void* host,
                    bool to_host, hipStream_t stream) {
    char* h = static_cast<char*>(host);
    auto one = [&](char* mem, size_t bytes, char* hp) {
        return to_host ? hipMemcpyAsync(hp, mem, bytes, hipMemcpyDefault, stream)
                       : hipMemcpyAsync(mem, hp, bytes, hipMemcpyDefault, stream);
    };
    hipError_t e = hipSuccess;
    if (b.flat) {
        e = one(static_cast<char*>(b.flat) + lo * es, static_cast<size_t>(hi - lo) * es, h);
    } else {
        int64_t t = std::upper_bound(p->prefix.begin(), p->prefix.end(), lo) - p->prefix.begin() - 1;
        for (int64_t x = lo; x < hi && e == hipSuccess; ++t) {
            const int64_t te = std::min(hi, p->prefix[t + 1]);
            if (te > x)
                e = one(static_cast<char*>(b.tensors[t]) + (x - p->prefix[t]) * es, static_cast<size_t>(te - x) * es,
                        h + (x - lo) * es);
            x = std::max(x, te);
        }
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return e == hipSuccess ? DP_OK : hip_fail(e, to_host ? "checkpoint copy to the host" : "checkpoint copy to the device");
}

dp_layout plan_layout(const dp_plan* p) {
    dp_layout L;
    std::memset(&L, 0, sizeof(L));
    L.num_tensors = p->T;
    L.n_replicas = p->n;
    L.numel = p->numel.data();
    L.grad_dtype = p->gdt;
    L.param_dtype = p->pdt;
    L.chunk_elems = p->chunk;
    return L;
}

dp_status read_device_state(dp_plan* p, hipStream_t stream, dpk::DevState* out) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpy(out, p->state, sizeof(*out), hipMemcpyDeviceToHost);
    return e == hipSuccess ? DP_OK : hip_fail(e, "reading the device state");
}

const dpapi::Binding* state_binding(const dp_plan* p, int array, int bank) {
    static const dp_role roles[kArrays] = {DP_ROLE_MASTER, DP_ROLE_EXP_AVG, DP_ROLE_EXP_AVG_SQ, DP_ROLE_PARAM};
    return &p->roles[roles[array]][array < 3 ? bank : 0];
}

dp_status device_checks(dp_plan* p, const char* dir, const char* where, int bank) {
    if (!p || !dir) return fail(DP_ERR_INVALID_ARG, "%s: null argument", where);
    if (!p->state_ready) return fail(DP_ERR_STATE, "%s before dp_state_init", where);
    static const char* const names[kArrays] = {"MASTER", "EXP_AVG", "EXP_AVG_SQ", "PARAM"};
    for (int a = 0; a < kArrays; ++a)
        if (!state_binding(p, a, bank)->bound)
            return fail(DP_ERR_UNBOUND, "%s: role %s (bank %d) is not bound", where, names[a], a < 3 ? bank : 0);
    return dpapi::ensure_device(p);
}

}  // namespace

extern "C" {

dp_status dp_ckpt_write_shard(const char* dir, int64_t generation, const dp_layout* layout, int64_t begin,
                              int64_t end, const float* master, const float* exp_avg, const float* exp_avg_sq,
                              const void* param) {
    dp_status s = check_layout(layout, "dp_ckpt_write_shard");
    if (s != DP_OK) return s;
    if (!dir || (end > begin && (!master || !exp_avg || !exp_avg_sq || !param)))
        return fail(DP_ERR_INVALID_ARG, "dp_ckpt_write_shard: null argument");
    const void* src[kArrays] = {master, exp_avg, exp_avg_sq, param};
    return write_shard(dir, generation, layout, begin, end, nullptr,
                       [&](int a, int64_t lo, int64_t, void*, const void** out) {
                           *out = static_cast<const char*>(src[a]) + (lo - begin) * esize(a, layout->param_dtype);
                           return DP_OK;
                       });
}

dp_status dp_ckpt_commit(const char* dir, int64_t generation, const dp_layout* layout, const dp_step_state* scalars,
                         const dp_state_cfg* cfg) {
    dp_status s = check_layout(layout, "dp_ckpt_commit");
    if (s != DP_OK) return s;
    if (!dir || !scalars || !cfg) return fail(DP_ERR_INVALID_ARG, "dp_ckpt_commit: null argument");
    return commit(dir, generation, layout, scalars, cfg);
}

dp_status dp_ckpt_read(const char* dir, const dp_layout* layout, int64_t begin, int64_t end, float* master,
                       float* exp_avg, float* exp_avg_sq, void* param, dp_step_state* scalars, dp_state_cfg* cfg,
                       int64_t* generation) {
    dp_status s = check_layout(layout, "dp_ckpt_read");
    if (s != DP_OK) return s;
    if (!dir) return fail(DP_ERR_INVALID_ARG, "dp_ckpt_read: null directory");
    void* dst[kArrays] = {master, exp_avg, exp_avg_sq, param};
    bool want[kArrays];
    for (int a = 0; a < kArrays; ++a) want[a] = dst[a] != nullptr;
    std::unique_ptr<char[]> staging(new (std::nothrow) char[read_staging_bytes(begin, end)]);
    if (!staging) return fail(DP_ERR_OOM, "dp_ckpt_read: host allocation of the staging buffer failed");
    return read_range(dir, layout, begin, end, staging.get(),
                      [&](int a, int64_t lo, int64_t hi, const void* src) {
                          const size_t es = esize(a, layout->param_dtype);
                          std::memcpy(static_cast<char*>(dst[a]) + (lo - begin) * es, src,
                                      static_cast<size_t>(hi - lo) * es);
                          return DP_OK;
                      },
                      want, scalars, cfg, generation);
}

dp_status dp_checkpoint_save(dp_plan* p, const char* dir, int64_t generation, int64_t begin, int64_t end,
                             hipStream_t stream) {
    if (!p || !dir) return fail(DP_ERR_INVALID_ARG, "dp_checkpoint_save: null argument");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_checkpoint_save before dp_state_init");
    dp_status s = dpapi::ensure_device(p);
    if (s != DP_OK) return s;
    dpk::DevState st;
    s = read_device_state(p, stream, &st);
    if (s != DP_OK) return s;
    const int bank = st.bank;
    s = device_checks(p, dir, "dp_checkpoint_save", bank);
    if (s != DP_OK) return s;
    Pinned stage;
    s = alloc_pinned(&stage, save_staging_bytes(begin, end));
    if (s != DP_OK) return s;
    const dp_layout L = plan_layout(p);
    return write_shard(dir, generation, &L, begin, end, stage.p,
                       [&](int a, int64_t lo, int64_t hi, void* staging, const void** out) {
                           *out = staging;
                           return copy_role(p, *state_binding(p, a, bank), esize(a, p->pdt), lo, hi, staging, true,
                                            stream);
                       });
}

dp_status dp_checkpoint_commit(dp_plan* p, const char* dir, int64_t generation, hipStream_t stream) {
    if (!p || !dir) return fail(DP_ERR_INVALID_ARG, "dp_checkpoint_commit: null argument");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_checkpoint_commit before dp_state_init");
    dp_status s = dpapi::ensure_device(p);
    if (s != DP_OK) return s;
    dpk::DevState st;
    s = read_device_state(p, stream, &st);
    if (s != DP_OK) return s;
    dp_step_state scalars;
    std::memcpy(&scalars, &st, sizeof(scalars));
    const dp_layout L = plan_layout(p);
    return commit(dir, generation, &L, &scalars, &p->cfg);
}

dp_status dp_checkpoint_load(dp_plan* p, const char* dir, int64_t begin, int64_t end, int32_t restore_scalars,
                             hipStream_t stream) {
    if (!p || !dir) return fail(DP_ERR_INVALID_ARG, "dp_checkpoint_load: null argument");
    if (!p->state_ready) return fail(DP_ERR_STATE, "dp_checkpoint_load before dp_state_init");
    dp_status s = dpapi::ensure_device(p);
    if (s != DP_OK) return s;
    // the range goes into the current bank, so the rest of the state stays
    // valid whether or not the caller restores it too
    dpk::DevState st;
    s = read_device_state(p, stream, &st);
    if (s != DP_OK) return s;
    const int bank = st.bank;
    s = device_checks(p, dir, "dp_checkpoint_load", bank);
    if (s != DP_OK) return s;
    const dp_layout L = plan_layout(p);
    dp_step_state saved;
    dp_state_cfg cfg;
    bool want[kArrays] = {false, false, false, false};
    const PutFn none = [](int, int64_t, int64_t, const void*) { return DP_OK; };
    // the manifest alone first (an empty range reads no shard): a layout or
    // settings mismatch fails before any of the plan's memory is written
    int64_t gen0 = 0, gen1 = 0;
    s = read_range(dir, &L, begin, begin, nullptr, none, want, &saved, &cfg, &gen0);
    if (s != DP_OK) return s;
    if (restore_scalars) {
        const dp_state_cfg& c = p->cfg;
        if (cfg.beta1 != c.beta1 || cfg.beta2 != c.beta2 || cfg.scaler_mode != c.scaler_mode ||
            (c.scaler_mode == DP_SCALER_DYNAMIC &&
             (cfg.growth_interval != c.growth_interval || cfg.backoff != c.backoff || cfg.growth != c.growth)))
            return fail(DP_ERR_STATE, "the checkpoint was taken with other optimizer settings (betas or loss scaler)");
    }
    Pinned stage;
    s = alloc_pinned(&stage, read_staging_bytes(begin, end));
    if (s != DP_OK) return s;
    std::fill(want, want + kArrays, true);
    s = read_range(dir, &L, begin, end, stage.p,
                   [&](int a, int64_t lo, int64_t hi, const void* src) {
                       return copy_role(p, *state_binding(p, a, bank), esize(a, p->pdt), lo, hi,
                                        const_cast<void*>(src), false, stream);
                   },
                   want, &saved, &cfg, &gen1);
    if (s != DP_OK) return s;
    if (gen1 != gen0)
        return fail(DP_ERR_STATE, "generation %lld was committed in %s during the load (it began at generation %lld)",
                    static_cast<long long>(gen1), dir, static_cast<long long>(gen0));
    if (restore_scalars) std::memcpy(&st, &saved, sizeof(st));
    st.bank = bank;
    hipError_t e = hipMemcpy(p->state, &st, sizeof(st), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "writing the device state");
    std::fill(p->micro.begin(), p->micro.end(), 0);
    p->partials_valid = false;
    p->stats_current = false;
    p->buckets.clear();
    p->bucket_elems = 0;
    p->bucket_mode = 0;
    return DP_OK;
}

}  // extern "C"
