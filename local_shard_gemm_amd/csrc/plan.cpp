// Host planner of libshardmm: meshes, partition specs, the four-case
// classification and per-rank / per-unit coordinates.
//
// Rules (page, section): one mesh axis shards at most one dimension of an
// array, and an unmentioned axis replicates it (lingze.zone "Notation";
// learntpu.dev ch05 "Notation"); the four cases from which operands shard
// the contracted dimension J (lingze.zone "Case 1".."Case 4", "Summary";
// learntpu.dev ch05 "The four cases of a sharded matmul"); the unreduced
// {U_axis} state of case-3 outputs (learntpu.dev ch05 Notation table).
#include <cctype>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

#ifndef SM_SOURCE_DIGEST
#define SM_SOURCE_DIGEST "unknown"
#endif

namespace shardmm {

// The build's source digest behind a fixed marker, so that the binding can
// read it from the file before loading the library.
static const char kBuildDigest[] = "SM_SOURCE_DIGEST=" SM_SOURCE_DIGEST;

static thread_local std::string g_last_error;

int32_t fail(int32_t status, const std::string& msg) {
  g_last_error = std::string(sm_status_str(status)) + ": " + msg;
  return status;
}

void clear_error() { g_last_error.clear(); }

size_t dtype_size(int32_t dt) { return dt == SM_BF16 ? 2 : dt == SM_F32 ? 4 : 0; }

int32_t axes_product(const sm_mesh& mesh, const int32_t* axes, int32_t n) {
  int32_t p = 1;
  for (int32_t i = 0; i < n; ++i) p *= mesh.sizes[axes[i]];
  return p;
}

int32_t block_of(const sm_mesh& mesh, const int32_t* axes, int32_t n, const int32_t* coords) {
  int32_t idx = 0;
  for (int32_t i = 0; i < n; ++i) idx = idx * mesh.sizes[axes[i]] + coords[axes[i]];
  return idx;
}

void rank_coords(const sm_mesh& mesh, int32_t rank, int32_t* coords) {
  for (int32_t a = mesh.n_axes - 1; a >= 0; --a) {
    coords[a] = rank % mesh.sizes[a];
    rank /= mesh.sizes[a];
  }
}

// Spread a flattened block index back over its axes (first listed = major).
static void unflatten(const sm_mesh& mesh, const int32_t* axes, int32_t n, int32_t idx,
                      int32_t* coords) {
  for (int32_t i = n - 1; i >= 0; --i) {
    int32_t s = mesh.sizes[axes[i]];
    coords[axes[i]] = idx % s;
    idx /= s;
  }
}

// A plan is trusted only if it is exactly what sm_plan makes of its own
// inputs (mesh, specs, sizes, dtypes): a plan edited after the fact could
// otherwise carry zero divisors or shapes that disagree with its views.
int32_t check_plan(const sm_plan_t* p) {
  if (!p) return fail(SM_ERR_ARG, "plan is NULL");
  if (p->magic != kPlanMagic) return fail(SM_ERR_ARG, "plan was not filled by sm_plan");
  sm_plan_t q;
  if (sm_plan(&p->mesh, &p->a, &p->b, p->I, p->J, p->K, p->in_dtype, p->out_dtype, &q) != SM_OK ||
      std::memcmp(&q, p, sizeof q) != 0)
    return fail(SM_ERR_ARG, "plan was modified after sm_plan");
  return SM_OK;
}

int32_t unit_view(const sm_plan_t& p, int32_t unit, UnitView* v) {
  if (p.kase != SM_CASE1 && p.kase != SM_CASE3)
    return fail(SM_ERR_NEEDS_GATHER, "case " + std::to_string(p.kase) + " has no local product");
  if (unit < 0 || unit >= p.n_units) return fail(SM_ERR_ARG, "unit out of range");
  int32_t coords[SM_MAX_AXES] = {0, 0, 0, 0};
  const int32_t g = unit / p.n_partials, y = unit % p.n_partials;
  const int32_t bi = g / p.c_grid[1], bk = g % p.c_grid[1];
  unflatten(p.mesh, p.a.axes[0], p.a.n[0], bi, coords);
  unflatten(p.mesh, p.b.axes[1], p.b.n[1], bk, coords);
  if (p.kase == SM_CASE3) unflatten(p.mesh, p.a.axes[1], p.a.n[1], y, coords);
  v->a_block[0] = block_of(p.mesh, p.a.axes[0], p.a.n[0], coords);
  v->a_block[1] = block_of(p.mesh, p.a.axes[1], p.a.n[1], coords);
  v->b_block[0] = block_of(p.mesh, p.b.axes[0], p.b.n[0], coords);
  v->b_block[1] = block_of(p.mesh, p.b.axes[1], p.b.n[1], coords);
  v->c_block[0] = bi;
  v->c_block[1] = bk;
  v->a_row0 = v->a_block[0] * p.a_local[0];
  v->a_col0 = v->a_block[1] * p.a_local[1];
  v->b_row0 = v->b_block[0] * p.b_local[0];
  v->b_col0 = v->b_block[1] * p.b_local[1];
  v->c_row0 = bi * p.c_local[0];
  v->c_col0 = bk * p.c_local[1];
  v->group = g;
  v->partial = y;
  return SM_OK;
}

// ------------------------------------------------------------ spec parsing

namespace {

struct Parser {
  const sm_mesh* mesh;
  std::string s;
  size_t i = 0;

  void ws() {
    while (i < s.size() && std::isspace(static_cast<unsigned char>(s[i]))) ++i;
  }
  bool eat(char c) {
    ws();
    if (i < s.size() && s[i] == c) {
      ++i;
      return true;
    }
    return false;
  }
  bool eat_word(const char* w) {
    ws();
    size_t n = std::strlen(w);
    if (s.compare(i, n, w) == 0 && (i + n == s.size() || !std::isalnum(static_cast<unsigned char>(s[i + n])))) {
      i += n;
      return true;
    }
    return false;
  }
  int32_t axis_index(const std::string& name) const {
    for (int32_t a = 0; a < mesh->n_axes; ++a)
      if (name == mesh->names[a]) return a;
    return -1;
  }
  // 'name' or "name"
  int32_t quoted(std::vector<int32_t>* out) {
    ws();
    if (i >= s.size() || (s[i] != '\'' && s[i] != '"')) return fail(SM_ERR_SPEC, "expected a quoted axis name");
    char q = s[i++];
    size_t j = s.find(q, i);
    if (j == std::string::npos) return fail(SM_ERR_SPEC, "unterminated axis name");
    std::string name = s.substr(i, j - i);
    i = j + 1;
    int32_t a = axis_index(name);
    if (a < 0) return fail(SM_ERR_SPEC, "unknown axis '" + name + "'");
    out->push_back(a);
    return SM_OK;
  }
  // None | 'X' | ('X', 'Y', ...)
  int32_t entry(std::vector<int32_t>* out) {
    if (eat_word("None")) return SM_OK;
    if (eat('(')) {
      if (eat(')')) return SM_OK;
      while (true) {
        int32_t st = quoted(out);
        if (st) return st;
        if (eat(')')) return SM_OK;
        if (!eat(',')) return fail(SM_ERR_SPEC, "expected ',' or ')' in axis tuple");
        if (eat(')')) return SM_OK;
      }
    }
    return quoted(out);
  }
};

}  // namespace

}  // namespace shardmm

using namespace shardmm;

extern "C" {

int32_t sm_abi_version(void) { return SM_ABI_VERSION; }
size_t sm_plan_size(void) { return sizeof(sm_plan_t); }

const char* sm_status_str(int32_t st) {
  switch (st) {
    case SM_OK: return "SM_OK";
    case SM_ERR_ARG: return "SM_ERR_ARG";
    case SM_ERR_MESH: return "SM_ERR_MESH";
    case SM_ERR_SPEC: return "SM_ERR_SPEC";
    case SM_ERR_AXIS_REUSED: return "SM_ERR_AXIS_REUSED";
    case SM_ERR_SHAPE: return "SM_ERR_SHAPE";
    case SM_ERR_INDIVISIBLE: return "SM_ERR_INDIVISIBLE";
    case SM_ERR_J_MISMATCH: return "SM_ERR_J_MISMATCH";
    case SM_ERR_NEEDS_GATHER: return "SM_ERR_NEEDS_GATHER";
    case SM_ERR_UNREDUCED: return "SM_ERR_UNREDUCED";
    case SM_ERR_CASE: return "SM_ERR_CASE";
    case SM_ERR_DTYPE: return "SM_ERR_DTYPE";
    case SM_ERR_ALIGN: return "SM_ERR_ALIGN";
    case SM_ERR_HIP: return "SM_ERR_HIP";
    default: return "SM_ERR_UNKNOWN";
  }
}

const char* sm_last_error(void) { return g_last_error.c_str(); }

int32_t sm_mesh_init(sm_mesh* mesh, int32_t n_axes, const char* const* names, const int32_t* sizes) {
  clear_error();
  if (!mesh || !names || !sizes) return fail(SM_ERR_ARG, "NULL argument");
  if (n_axes < 1 || n_axes > SM_MAX_AXES) return fail(SM_ERR_MESH, "1 to 4 axes");
  std::memset(mesh, 0, sizeof *mesh);
  mesh->n_axes = n_axes;
  for (int32_t a = 0; a < n_axes; ++a) {
    if (!names[a]) return fail(SM_ERR_MESH, "NULL axis name");
    size_t len = std::strlen(names[a]);
    if (len == 0 || len >= SM_NAME_LEN) return fail(SM_ERR_MESH, "axis names are 1..7 characters");
    for (size_t c = 0; c < len; ++c)
      if (!std::isalnum(static_cast<unsigned char>(names[a][c])) && names[a][c] != '_')
        return fail(SM_ERR_MESH, "axis names are alphanumeric");
    if (sizes[a] < 1) return fail(SM_ERR_MESH, "axis sizes must be >= 1");
    std::memcpy(mesh->names[a], names[a], len);
    mesh->sizes[a] = sizes[a];
    for (int32_t b = 0; b < a; ++b)
      if (std::strcmp(mesh->names[a], mesh->names[b]) == 0) return fail(SM_ERR_MESH, "duplicate axis name");
  }
  int64_t ranks = 1;
  for (int32_t a = 0; a < n_axes; ++a) ranks *= sizes[a];
  if (ranks > (1 << 20)) return fail(SM_ERR_MESH, "more than 2^20 ranks");
  return SM_OK;
}

int32_t sm_parse_spec(const sm_mesh* mesh, const char* text, sm_spec* out) {
  clear_error();
  if (!mesh || !text || !out) return fail(SM_ERR_ARG, "NULL argument");
  if (mesh->n_axes < 1 || mesh->n_axes > SM_MAX_AXES) return fail(SM_ERR_MESH, "bad mesh");
  Parser ps{mesh, std::string(text)};
  std::vector<int32_t> dims[2];
  int32_t ndims = 0;
  std::string t = ps.s;
  // trim
  size_t b = t.find_first_not_of(" \t\r\n"), e = t.find_last_not_of(" \t\r\n");
  t = (b == std::string::npos) ? std::string() : t.substr(b, e - b + 1);
  std::memset(out, 0, sizeof *out);
  if (t.empty() || t == "None") return SM_OK;

  const bool quotedq = t.find('\'') != std::string::npos || t.find('"') != std::string::npos;
  const size_t lb = t.find('[');
  const bool bracketed = lb != std::string::npos && t.back() == ']';
  if (bracketed || (!quotedq && t[0] != 'P' && t.find("None") == std::string::npos)) {
    // Subscript notation: A[I_X, J_YZ] or I_X, J (single-letter axis names).
    std::string body = bracketed ? t.substr(lb + 1, t.size() - lb - 2) : t;
    size_t pos = 0;
    while (true) {
      size_t comma = body.find(',', pos);
      std::string part = body.substr(pos, comma == std::string::npos ? std::string::npos : comma - pos);
      if (ndims >= 2) return fail(SM_ERR_SPEC, "more than 2 dimensions");
      size_t p0 = part.find_first_not_of(" \t"), p1 = part.find_last_not_of(" \t");
      if (p0 == std::string::npos) return fail(SM_ERR_SPEC, "empty dimension");
      part = part.substr(p0, p1 - p0 + 1);
      size_t us = part.find('_');
      for (size_t c = 0; c < (us == std::string::npos ? part.size() : us); ++c)
        if (!std::isalpha(static_cast<unsigned char>(part[c]))) return fail(SM_ERR_SPEC, "bad dimension name");
      if (us != std::string::npos) {
        std::string sub = part.substr(us + 1);
        if (sub.empty()) return fail(SM_ERR_SPEC, "empty subscript");
        for (char ch : sub) {
          int32_t a = ps.axis_index(std::string(1, ch));
          if (a < 0) return fail(SM_ERR_SPEC, std::string("unknown axis '") + ch + "'");
          dims[ndims].push_back(a);
        }
      }
      ++ndims;
      if (comma == std::string::npos) break;
      pos = comma + 1;
    }
  } else {
    ps.s = t;
    ps.i = 0;
    bool has_p = false;
    if (ps.eat('P')) {
      if (!ps.eat('(')) return fail(SM_ERR_SPEC, "expected '(' after P");
      has_p = true;
    }
    ps.ws();
    bool empty = has_p ? ps.eat(')') : false;
    while (!empty) {
      if (ndims >= 2) return fail(SM_ERR_SPEC, "more than 2 dimensions");
      int32_t st = ps.entry(&dims[ndims]);
      if (st) return st;
      ++ndims;
      if (has_p && ps.eat(')')) break;
      if (!ps.eat(',')) {
        ps.ws();
        if (!has_p && ps.i >= ps.s.size()) break;
        return fail(SM_ERR_SPEC, "expected ','");
      }
      if (has_p && ps.eat(')')) break;
      ps.ws();
      if (!has_p && ps.i >= ps.s.size()) break;
    }
    ps.ws();
    if (ps.i != ps.s.size()) return fail(SM_ERR_SPEC, "trailing characters in spec");
  }
  for (int32_t d = 0; d < 2; ++d) {
    if (dims[d].size() > SM_MAX_AXES) return fail(SM_ERR_AXIS_REUSED, "axis repeated");
    out->n[d] = static_cast<int32_t>(dims[d].size());
    for (size_t k = 0; k < dims[d].size(); ++k) out->axes[d][k] = dims[d][k];
  }
  return SM_OK;
}

static int32_t validate_spec_impl(const sm_mesh& mesh, const sm_spec& s, const char* what) {
  uint32_t used = 0;
  for (int32_t d = 0; d < 2; ++d) {
    if (s.n[d] < 0 || s.n[d] > SM_MAX_AXES) return fail(SM_ERR_SPEC, std::string(what) + ": bad axis count");
    for (int32_t k = 0; k < s.n[d]; ++k) {
      int32_t a = s.axes[d][k];
      if (a < 0 || a >= mesh.n_axes) return fail(SM_ERR_SPEC, std::string(what) + ": axis index out of range");
      if (used & (1u << a))
        return fail(SM_ERR_AXIS_REUSED, std::string(what) + ": axis '" + mesh.names[a] + "' shards two dimensions");
      used |= 1u << a;
    }
  }
  return SM_OK;
}

static uint32_t spec_mask(const sm_spec& s) {
  uint32_t m = 0;
  for (int32_t d = 0; d < 2; ++d)
    for (int32_t k = 0; k < s.n[d]; ++k) m |= 1u << s.axes[d][k];
  return m;
}

static uint32_t dim_mask(const sm_spec& s, int32_t d) {
  uint32_t m = 0;
  for (int32_t k = 0; k < s.n[d]; ++k) m |= 1u << s.axes[d][k];
  return m;
}

static int32_t copies_outside(const sm_mesh& mesh, uint32_t used) {
  int32_t c = 1;
  for (int32_t a = 0; a < mesh.n_axes; ++a)
    if (!(used & (1u << a))) c *= mesh.sizes[a];
  return c;
}

static int32_t split(int64_t total, const sm_mesh& mesh, const int32_t* axes, int32_t n, const char* what,
                     int64_t* local, int32_t* parts) {
  int32_t p = axes_product(mesh, axes, n);
  if (total % p) return fail(SM_ERR_INDIVISIBLE, std::string(what) + " does not split evenly");
  *local = total / p;
  *parts = p;
  return SM_OK;
}

int32_t sm_plan(const sm_mesh* mesh, const sm_spec* a, const sm_spec* b, int64_t I, int64_t J, int64_t K,
                int32_t in_dtype, int32_t out_dtype, sm_plan_t* out) {
  clear_error();
  if (!mesh || !a || !b || !out) return fail(SM_ERR_ARG, "NULL argument");
  if (mesh->n_axes < 1 || mesh->n_axes > SM_MAX_AXES) return fail(SM_ERR_MESH, "1 to 4 axes");
  int64_t ranks = 1;
  for (int32_t x = 0; x < mesh->n_axes; ++x) {
    if (mesh->sizes[x] < 1) return fail(SM_ERR_MESH, "axis sizes must be >= 1");
    ranks *= mesh->sizes[x];
    if (ranks > kMaxRanks) return fail(SM_ERR_MESH, "more than 2^20 ranks");
  }
  int32_t st;
  if ((st = validate_spec_impl(*mesh, *a, "A"))) return st;
  if ((st = validate_spec_impl(*mesh, *b, "B"))) return st;
  if (I < 1 || J < 1 || K < 1) return fail(SM_ERR_SHAPE, "I, J and K must be >= 1");
  if (I > (int64_t(1) << 40) || J > (int64_t(1) << 40) || K > (int64_t(1) << 40))
    return fail(SM_ERR_SHAPE, "dimension too large");
  if (in_dtype != SM_BF16) return fail(SM_ERR_DTYPE, "inputs must be bfloat16");
  if (out_dtype != SM_F32 && out_dtype != SM_BF16) return fail(SM_ERR_DTYPE, "output must be float32 or bfloat16");

  sm_plan_t p;
  std::memset(&p, 0, sizeof p);
  p.mesh = *mesh;
  p.a = *a;
  p.b = *b;
  p.I = I;
  p.J = J;
  p.K = K;
  p.in_dtype = in_dtype;
  p.out_dtype = out_dtype;
  p.n_ranks = 1;
  for (int32_t x = 0; x < mesh->n_axes; ++x) p.n_ranks *= mesh->sizes[x];

  int64_t bk_rows = 0;
  if ((st = split(I, *mesh, a->axes[0], a->n[0], "A rows (I)", &p.a_local[0], &p.a_grid[0]))) return st;
  if ((st = split(J, *mesh, a->axes[1], a->n[1], "A cols (J)", &p.a_local[1], &p.a_grid[1]))) return st;
  if ((st = split(J, *mesh, b->axes[0], b->n[0], "B rows (J)", &bk_rows, &p.b_grid[0]))) return st;
  if ((st = split(K, *mesh, b->axes[1], b->n[1], "B cols (K)", &p.b_local[1], &p.b_grid[1]))) return st;
  p.b_local[0] = bk_rows;
  p.a_copies = copies_outside(*mesh, spec_mask(*a));
  p.b_copies = copies_outside(*mesh, spec_mask(*b));

  const uint32_t a_i = dim_mask(*a, 0), a_j = dim_mask(*a, 1);
  const uint32_t b_j = dim_mask(*b, 0), b_k = dim_mask(*b, 1);
  p.gather_operand = -1;
  if (a_i & b_k) {
    // Case 4: a shared axis on the non-contracting dims; only diagonal blocks
    // are formed. Fix by gathering the smaller operand over the shared axes.
    p.kase = SM_CASE4;
    p.gather_operand = I <= K ? 0 : 1;  // bytes I*J vs J*K (J >= 1), without the product
    p.gather_axes = a_i & b_k;
  } else if (a->n[1] > 0 && b->n[0] > 0) {
    bool same = a->n[1] == b->n[0];
    for (int32_t k = 0; same && k < a->n[1]; ++k) same = a->axes[1][k] == b->axes[0][k];
    if (!same) return fail(SM_ERR_J_MISMATCH, "A and B shard J over different axes");
    p.kase = SM_CASE3;
    p.reduce_axes = a_j;
  } else if (a->n[1] > 0 || b->n[0] > 0) {
    p.kase = SM_CASE2;
    p.gather_operand = a->n[1] > 0 ? 0 : 1;
    p.gather_axes = a->n[1] > 0 ? a_j : b_j;
  } else {
    p.kase = SM_CASE1;
  }
  if (p.kase == SM_CASE3 && out_dtype != SM_F32)
    return fail(SM_ERR_DTYPE, "partial sums are stored in float32");

  p.c_local[0] = p.a_local[0];
  p.c_local[1] = p.b_local[1];
  p.c_grid[0] = p.a_grid[0];
  p.c_grid[1] = p.b_grid[1];
  p.n_partials = p.kase == SM_CASE3 ? axes_product(*mesh, a->axes[1], a->n[1]) : 1;
  p.n_groups = p.c_grid[0] * p.c_grid[1];
  p.n_units = p.n_groups * p.n_partials;
  p.c_copies = copies_outside(*mesh, a_i | b_k | p.reduce_axes);

  p.c.n[0] = a->n[0];
  p.c.n[1] = b->n[1];
  for (int32_t k = 0; k < a->n[0]; ++k) p.c.axes[0][k] = a->axes[0][k];
  for (int32_t k = 0; k < b->n[1]; ++k) p.c.axes[1][k] = b->axes[1][k];
  if (p.kase == SM_CASE3) {
    // After reduce-scatter the reduced axes split the rows as minor axes.
    p.c_rs = p.c;
    for (int32_t k = 0; k < a->n[1]; ++k) p.c_rs.axes[0][p.c_rs.n[0]++] = a->axes[1][k];
  }
  p.magic = kPlanMagic;
  std::memcpy(out, &p, sizeof p);  // padding bytes included: check_plan compares bytes
  return SM_OK;
}

int32_t sm_plan_gathered(const sm_plan_t* plan, sm_plan_t* out) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  if (!out) return fail(SM_ERR_ARG, "NULL output");
  if (plan->kase != SM_CASE2 && plan->kase != SM_CASE4)
    return fail(SM_ERR_CASE, "only case-2 and case-4 plans need an operand gathered");
  // The gathered operand loses the gather axes from both of its dims.
  sm_spec a = plan->a, b = plan->b;
  sm_spec& g = plan->gather_operand == 0 ? a : b;
  for (int32_t d = 0; d < 2; ++d) {
    int32_t kept = 0;
    for (int32_t k = 0; k < g.n[d]; ++k)
      if (!(plan->gather_axes & (1u << g.axes[d][k]))) g.axes[d][kept++] = g.axes[d][k];
    for (int32_t k = kept; k < SM_MAX_AXES; ++k) g.axes[d][k] = 0;
    g.n[d] = kept;
  }
  sm_plan_t q;
  if ((st = sm_plan(&plan->mesh, &a, &b, plan->I, plan->J, plan->K, plan->in_dtype, plan->out_dtype, &q)))
    return st;
  *out = q;  // case 1 or 3; case 2 again when the other operand is J-sharded
  return SM_OK;
}

int32_t sm_rank_info(const sm_plan_t* plan, int32_t rank, sm_rank_info_t* out) {
  clear_error();
  int32_t st = check_plan(plan);
  if (st) return st;
  if (!out) return fail(SM_ERR_ARG, "NULL output");
  if (rank < 0 || rank >= plan->n_ranks) return fail(SM_ERR_ARG, "rank out of range");
  const sm_plan_t& p = *plan;
  sm_rank_info_t r;
  std::memset(&r, 0, sizeof r);
  rank_coords(p.mesh, rank, r.coords);
  r.a_block[0] = block_of(p.mesh, p.a.axes[0], p.a.n[0], r.coords);
  r.a_block[1] = block_of(p.mesh, p.a.axes[1], p.a.n[1], r.coords);
  r.b_block[0] = block_of(p.mesh, p.b.axes[0], p.b.n[0], r.coords);
  r.b_block[1] = block_of(p.mesh, p.b.axes[1], p.b.n[1], r.coords);
  r.c_block[0] = r.a_block[0];
  r.c_block[1] = r.b_block[1];
  r.a_row0 = r.a_block[0] * p.a_local[0];
  r.a_col0 = r.a_block[1] * p.a_local[1];
  r.b_row0 = r.b_block[0] * p.b_local[0];
  r.b_col0 = r.b_block[1] * p.b_local[1];
  r.c_row0 = r.c_block[0] * p.c_local[0];
  r.c_col0 = r.c_block[1] * p.c_local[1];
  r.rs_row0 = -1;
  r.rs_rows = 0;
  if (p.kase == SM_CASE1 || p.kase == SM_CASE3) {
    r.group = r.c_block[0] * p.c_grid[1] + r.c_block[1];
    r.partial = p.kase == SM_CASE3 ? r.a_block[1] : 0;
    r.unit = r.group * p.n_partials + r.partial;
    if (p.kase == SM_CASE3 && p.c_local[0] % p.n_partials == 0) {
      r.rs_rows = p.c_local[0] / p.n_partials;
      r.rs_row0 = r.c_row0 + r.partial * r.rs_rows;
    }
  } else {
    r.unit = r.group = r.partial = -1;
  }
  *out = r;
  return SM_OK;
}

}  // extern "C"

int32_t shardmm::validate_spec(const sm_mesh& mesh, const sm_spec& s, const char* what) {
  return validate_spec_impl(mesh, s, what);
}

extern "C" const char* sm_build_digest(void) { return shardmm::kBuildDigest + sizeof("SM_SOURCE_DIGEST=") - 1; }
